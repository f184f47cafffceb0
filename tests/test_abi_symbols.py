"""The C-ABI library loads (no GPU needed) and exports every declared symbol."""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b(kvm_\w+)\s*\(", txt, flags=re.M))
    return names


def test_header_declares_the_four_calls_and_helpers():
    names = declared()
    for n in ("kvm_build_index", "kvm_score_blocks", "kvm_select", "kvm_rematerialize"):
        assert n in names
    assert len(names) >= 15


def test_library_loads_and_exports_every_declared_symbol():
    import attention_space_block_amd as k
    lib = k._abi.lib()
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", k.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(kvm_\w+)$", out, flags=re.M))
    assert declared() <= exported
    assert set(k.EXPORTED) == declared()
    assert k.kvm_version() == 104


def test_validation_errors_need_no_gpu():
    import attention_space_block_amd as k
    d = k.Dims(1, 2, 4, 96, 32)                       # unsupported head_dim
    try:
        k.kvm_build_index(d, k.KVM_F32, 16, 1 << 20, 0, 1, 16, 1, stream=0)
    except k.KvmError as e:
        assert e.code == -5
    else:
        raise AssertionError("expected KVM_ENOTSUP")
    d = k.Dims(1, 2, 4, 64, 32)
    try:                                              # range beyond capacity
        k.kvm_build_index(d, k.KVM_F32, 16, 1 << 20, 5, 10, 16, 8, stream=0)
    except k.KvmError as e:
        assert e.code == -1 and "capacity" in str(e)
    else:
        raise AssertionError("expected KVM_EINVAL")
    assert k.kvm_score_ws_bytes(d, k.KVM_F32, 1, 128) > 0
    try:
        k.kvm_select(16, 100, 50, 60, 100, 32, 16, 16, 16, stream=0)
    except k.KvmError as e:
        assert e.code == -4
    else:
        raise AssertionError("expected KVM_ERANGE")
    for args in ((16, 7, 100, 16), (16, k.KVM_BF16, 0, 16), (16, k.KVM_BF16, 100, 18),
                 (0, k.KVM_F32, 100, 16)):
        try:                                          # dtype, n, dst alignment, null src
            k.kvm_quantize_e4m3(*args, stream=0)
        except k.KvmError as e:
            assert e.code == -1
        else:
            raise AssertionError(f"expected KVM_EINVAL for {args}")
    # FP8 scores need d = 128 and either T*G <= 64 (stored path, either index
    # location) or an index in HBM (two-pass path)
    d = k.Dims(1, 2, 12, 128, 32)                    # G = 6
    assert k.kvm_score_ws_bytes(d, k.KVM_FP8_E4M3, 1, 256) > 0
    assert k.kvm_score_ws_bytes(d, k.KVM_FP8_E4M3, 16, 256) > 0
    assert k.kvm_score_ws_bytes(d, k.KVM_FP8_E4M3, 10, 1024, k.KVM_INDEX_HOST_TILED, 512) > 0
    assert k.kvm_score_ws_bytes(d, k.KVM_FP8_E4M3, 11, 1024, k.KVM_INDEX_HOST_TILED, 512) == 0
    assert k.kvm_score_ws_bytes(k.Dims(1, 2, 12, 64, 32), k.KVM_FP8_E4M3, 1, 256) == 0
