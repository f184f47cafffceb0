"""Thin ctypes binding of libkvm.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
turns tensors into pointers and checks return codes. Importing it fails
loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvm.so")

KVM_OK, KVM_EINVAL, KVM_ENOMEM, KVM_EHIP, KVM_ERANGE, KVM_ENOTSUP = 0, -1, -2, -3, -4, -5
KVM_EINTERNAL = -6
KVM_F32, KVM_BF16, KVM_FP8_E4M3 = 0, 1, 2
KVM_INDEX_DEVICE, KVM_INDEX_HOST_TILED = 0, 1
KVM_SRC_NONE, KVM_SRC_HOST_PINNED, KVM_SRC_DEVICE = 0, 1, 2
KVM_TIER_LRU, KVM_TIER_LRFU = 0, 1
KVM_RATE_COPY, KVM_RATE_MFMA_BF16, KVM_RATE_EXP, KVM_RATE_SCORE_MIX = 0, 1, 2, 3

EXPORTED = [
    "kvm_version", "kvm_last_error", "kvm_build_index", "kvm_score_ws_bytes", "kvm_score_blocks",
    "kvm_select_ws_bytes", "kvm_select", "kvm_select_noalloc", "kvm_ctx_create", "kvm_ctx_destroy",
    "kvm_ctx_set_source", "kvm_ctx_set_gather", "kvm_ctx_register_resident",
    "kvm_ctx_register_resident_list",
    "kvm_ctx_build_index_rope", "kvm_rematerialize", "kvm_ctx_sync", "kvm_ctx_set_serialized",
    "kvm_ctx_block_state",
    "kvm_ctx_block_deltas", "kvm_ctx_evict", "kvm_tier_simulate", "kvm_quantize_e4m3",
    "kvm_profile_enable", "kvm_profile_read", "kvm_measure_rate",
]


class KvmError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func} returned {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32)]


class CtxDesc(ctypes.Structure):
    _fields_ = [("dims", Dims), ("dtype", ctypes.c_int32), ("rope_layout", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("max_pos", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("k_view", ctypes.c_void_p),
                ("v_view", ctypes.c_void_p), ("k_shadow", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int64), ("batch_blocks", ctypes.c_int32),
                ("staging_blocks", ctypes.c_int32), ("delta_limit", ctypes.c_int32)]


class RematStats(ctypes.Structure):
    _fields_ = [("n_sel", ctypes.c_int32), ("hits", ctypes.c_int32), ("misses", ctypes.c_int32),
                ("rotated", ctypes.c_int32), ("evicted", ctypes.c_int32),
                ("batches", ctypes.c_int32), ("h2d_bytes", ctypes.c_int64),
                ("d2d_bytes", ctypes.c_int64), ("deltas", ctypes.c_int32),
                ("rebuilds", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class TierPolicy(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int32), ("host_blocks", ctypes.c_int32),
                ("lam", ctypes.c_double)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


GATHER_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                             ctypes.c_void_p)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz, f32p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p)
        dp = ctypes.POINTER(Dims)
        sig = {
            "kvm_version": (ctypes.c_int, []),
            "kvm_last_error": (ctypes.c_char_p, []),
            "kvm_build_index": (ctypes.c_int, [dp, i32, vp, i64, i64, i64, vp, i64, vp]),
            "kvm_score_ws_bytes": (sz, [dp, i32, i32, i64, i32, i64]),
            "kvm_score_blocks": (ctypes.c_int, [dp, i32, vp, i32, vp, i64, i64, i32, i64, f32p,
                                                vp, sz, vp]),
            "kvm_select_ws_bytes": (sz, [i64]),
            "kvm_select": (ctypes.c_int, [f32p, i64, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
            "kvm_select_noalloc": (ctypes.c_int, [f32p, i64, i32, i32, i32, i32, vp, vp, vp, vp]),
            "kvm_ctx_create": (ctypes.c_int, [ctypes.POINTER(CtxDesc), ctypes.POINTER(vp)]),
            "kvm_ctx_destroy": (None, [vp]),
            "kvm_ctx_set_source": (ctypes.c_int, [vp, i64, i64, vp, vp, i64, i32]),
            "kvm_ctx_set_gather": (ctypes.c_int, [vp, i64, i64, GATHER_FN, vp]),
            "kvm_ctx_register_resident": (ctypes.c_int, [vp, i64, i64, vp, vp, i64, vp]),
            "kvm_ctx_register_resident_list": (ctypes.c_int, [vp, vp, i64, vp, vp, i64, vp]),
            "kvm_measure_rate": (ctypes.c_int, [i32, i64, vp, sz, vp, vp]),
            "kvm_ctx_build_index_rope": (ctypes.c_int, [vp, vp, i64, i64, i64, i64, vp, i64, vp]),
            "kvm_rematerialize": (ctypes.c_int, [vp, vp, vp, vp, ctypes.POINTER(RematStats), vp]),
            "kvm_ctx_sync": (ctypes.c_int, [vp]),
            "kvm_ctx_set_serialized": (ctypes.c_int, [vp, ctypes.c_int32]),
            "kvm_ctx_block_state": (ctypes.c_int, [vp, i64, ctypes.POINTER(i32),
                                                   ctypes.POINTER(i32)]),
            "kvm_ctx_block_deltas": (ctypes.c_int, [vp, i64, ctypes.POINTER(i32)]),
            "kvm_ctx_evict": (ctypes.c_int, [vp, i64, i64]),
            "kvm_tier_simulate": (ctypes.c_int, [ctypes.POINTER(TierPolicy), i32, vp, vp, vp, vp,
                                                 vp, vp, vp]),
            "kvm_quantize_e4m3": (ctypes.c_int, [vp, i32, i64, vp, vp]),
            "kvm_profile_enable": (ctypes.c_int, [i32]),
            "kvm_profile_read": (ctypes.c_int, [ctypes.POINTER(KernelStat), i32,
                                                ctypes.POINTER(i32)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(rc: int, func: str) -> int:
    if rc != KVM_OK:
        raise KvmError(rc, func, lib().kvm_last_error().decode())
    return rc
