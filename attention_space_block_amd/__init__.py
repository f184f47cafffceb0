"""MI355X (gfx950) attention-space block retrieval and rematerialization.

The per-step working-set update of KVMem ("Virtualizing Million-Token Agent
Workspaces on a Consumer GPU", Sec. 4.2-4.4, Sec. 5) as a C-ABI library
(``libkvm.so``, declared in ``include/kvm.h``) of hand-written HIP kernels,
with this thin Python binding over it (same names as the C entry points).
PyTorch supplies device memory and streams only.
"""
from .api import (  # noqa: F401
    Dims, KvmCtx, KvmError, RematStats, dims_for, dtype_code, kvm_version, kvm_build_index,
    kvm_score_ws_bytes, kvm_score_blocks, kvm_select_ws_bytes, kvm_select, kvm_select_noalloc,
    kvm_profile_enable, kvm_profile_read, kvm_tier_simulate, kvm_quantize_e4m3,
    kvm_measure_rate, KVM_RATE_COPY, KVM_RATE_MFMA_BF16, KVM_RATE_EXP, KVM_RATE_SCORE_MIX,
    KVM_F32, KVM_BF16, KVM_FP8_E4M3, KVM_INDEX_DEVICE, KVM_INDEX_HOST_TILED,
    KVM_SRC_NONE, KVM_SRC_HOST_PINNED, KVM_SRC_DEVICE, KVM_TIER_LRU, KVM_TIER_LRFU,
)
from ._abi import EXPORTED, LIB_PATH  # noqa: F401
from .step import WorkingSetUpdater  # noqa: F401
