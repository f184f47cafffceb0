"""NumPy-facing wrappers over the compiled generator in gen.c."""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .workloads import TENSOR, Workload

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None


def default_threads() -> int:
    # One GPU's share of host cores is 16; never more.
    return max(1, min(16, os.cpu_count() or 1))


def build_library(force: bool = False) -> str:
    """Compile gen.c with gcc (no fused multiply-add, so bits are portable)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build_library()
            lib = ctypes.CDLL(_LIB_PATH)
            u64, i64, i32, f32, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_float, ctypes.c_void_p)
            lib.synth_key.restype = u64
            lib.synth_key.argtypes = [u64, u64, u64, u64]
            lib.synth_unit_f32.restype = None
            lib.synth_unit_f32.argtypes = [u64, u64, i64, vp]
            lib.synth_kv_blocks.restype = None
            lib.synth_kv_blocks.argtypes = [u64, i32, i32, f32, i64, i64, i32, i32, i32,
                                            i32, i32, vp, i64, i32]
            lib.synth_query.restype = None
            lib.synth_query.argtypes = [u64, i32, i32, i32, i32, i32, vp, i32, vp, i32]
            lib.synth_index_direct.restype = None
            lib.synth_index_direct.argtypes = [u64, i32, i32, f32, i64, i64, i64, i64, i32,
                                               vp, i64, i32]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_key(seed: int, tensor: int, i0: int, i1: int) -> int:
    return int(_load().synth_key(seed, tensor, i0, i1))


def unit_stream(key: int, e0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_unit_f32(key, e0, n, _ptr(out))
    return out


def _dtype_code(dtype: str) -> int:
    return {"f32": 0, "bf16": 1, "fp8": 2}[dtype]


def _np_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


def kv_blocks(wl: Workload, which: str, b0: int, nb: int, out: np.ndarray | None = None,
              nthreads: int | None = None) -> np.ndarray:
    """Raw K ("K") or V ("V") of blocks [b0, b0+nb), shape [nb][L][Hkv][B][d].

    bf16 data is returned as uint16 bit patterns; fp32 as float32. ``out`` may
    be any C-contiguous buffer of the right size (e.g. a pinned tensor's numpy
    view)."""
    shape = (nb, wl.n_layers, wl.n_kv_heads, wl.block_tokens, wl.head_dim)
    if out is None:
        out = np.empty(shape, dtype=_np_dtype(wl.dtype))
    assert out.nbytes == nb * wl.block_bytes
    tensor = TENSOR["K"] if which == "K" else TENSOR["V"]
    off_t = TENSOR["KOFF"] if which == "K" else TENSOR["VOFF"]
    _load().synth_kv_blocks(wl.seed, tensor, off_t, wl.off_sigma, b0, nb, wl.n_layers,
                            wl.n_kv_heads, wl.block_tokens, wl.head_dim,
                            _dtype_code(wl.dtype), _ptr(out), wl.block_bytes,
                            nthreads or default_threads())
    return out


_shift_cache: dict = {}


def churn_shift(wl: Workload, step: int) -> np.ndarray:
    """Query topic u(step) [L][Hq][d] fp32 of the churn workload.

    u(0) = s*w0; u(t) = rho*u(t-1) + (s*sqrt(1-rho^2))*w_t, each product and
    sum one fp32 operation, with w_t = unit(key(seed, WSTEP+t, l, h), dim)."""
    L, Hq, d = wl.n_layers, wl.n_q_heads, wl.head_dim
    rho = np.float32(wl.topic_rho)
    s = np.float32(wl.topic_scale)
    c = np.float32(wl.topic_scale * np.sqrt(1.0 - wl.topic_rho ** 2))

    def w(t):
        arr = np.empty((L, Hq, d), dtype=np.float32)
        for l in range(L):
            for h in range(Hq):
                arr[l, h] = unit_stream(stream_key(wl.seed, TENSOR["WSTEP"] + t, l, h), 0, d)
        return arr

    key = (wl.seed, L, Hq, d, wl.topic_rho, wl.topic_scale)
    t0, u = 0, (s * w(0)).astype(np.float32)
    for t in range(step, 0, -1):                 # resume from the latest cached step
        if (key, t) in _shift_cache:
            t0, u = t, _shift_cache[(key, t)]
            break
    for t in range(t0 + 1, step + 1):
        u = (rho * u).astype(np.float32) + (c * w(t)).astype(np.float32)
        u = u.astype(np.float32)
    _shift_cache[(key, step)] = u
    return u


def query(wl: Workload, step: int = 0, shift: np.ndarray | None = None,
          nthreads: int | None = None) -> np.ndarray:
    """Query vectors [L][Hq][T][d] (uint16 bf16 bits or float32).

    Single-step workloads draw from stream Q; the churn workload draws step t
    from QSTEP+t and adds the topic u(t). ``shift`` ([L][Hq][d] fp32) is added
    to every token when given (used to plant a direction)."""
    L, Hq, T, d = wl.n_layers, wl.n_q_heads, wl.n_q_tokens, wl.head_dim
    tensor = TENSOR["Q"]
    if wl.steps > 1:
        tensor = TENSOR["QSTEP"] + step
        if shift is None:
            shift = churn_shift(wl, step)
    out = np.empty((L, Hq, T, d), dtype=_np_dtype(wl.index_dtype))
    sp = None
    if shift is not None:
        shift = np.ascontiguousarray(shift, dtype=np.float32)
        assert shift.shape == (L, Hq, d)
        sp = _ptr(shift)
    _load().synth_query(wl.seed, tensor, L, Hq, T, d, sp, _dtype_code(wl.index_dtype), _ptr(out),
                        nthreads or default_threads())
    return out


def index_direct(wl: Workload, b0: int, nb: int, out: np.ndarray | None = None,
                 lg_stride_elems: int | None = None, nthreads: int | None = None,
                 lg0: int = 0, n_lg: int | None = None) -> np.ndarray:
    """A directly drawn bf16 index for blocks [b0, b0+nb) of (l, g) pairs
    [lg0, lg0+n_lg) (all pairs by default), rows flattened as l*Hkv + g.

    Default layout [L][Hkv][nb][d] (or [n_lg][nb][d] for a pair range); pass
    ``out``/``lg_stride_elems`` to write into a larger buffer or a tile."""
    L, Hkv, d = wl.n_layers, wl.n_kv_heads, wl.head_dim
    all_pairs = n_lg is None
    n_lg = L * Hkv if all_pairs else n_lg
    if out is None:
        shape = (L, Hkv, nb, d) if all_pairs and lg0 == 0 else (n_lg, nb, d)
        out = np.empty(shape, dtype=np.uint16)
        lg_stride_elems = nb * d
    _load().synth_index_direct(wl.seed, TENSOR["IDX"], TENSOR["KOFF"], wl.off_sigma, b0, nb,
                               lg0, n_lg, d, _ptr(out), lg_stride_elems,
                               nthreads or default_threads())
    return out


def scores_f32(seed: int, n: int, kind: str = "cont", levels: int = 8) -> np.ndarray:
    """Synthetic non-negative fp32 score vectors for selection tests.

    kind "cont": |unit|; "ties": floor(|unit|*levels)/levels (many exact ties);
    "const": all equal."""
    x = np.abs(unit_stream(stream_key(seed, TENSOR["SCORE"], n, 0), 0, n))
    if kind == "ties":
        x = (np.floor(x * np.float32(levels)) / np.float32(levels)).astype(np.float32)
    elif kind == "const":
        x = np.full(n, np.float32(0.25), dtype=np.float32)
    return x.astype(np.float32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit pattern (input-side storage)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


class _Store(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("off_sigma", ctypes.c_float),
                ("L", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("B", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def gather_store(wl: Workload):
    """(C function pointer, user pointer, keep-alive) of a generator-backed
    lower tier: the function writes any block's raw K or V on demand."""
    assert TENSOR["K"] == 1 and TENSOR["V"] == 2 and TENSOR["KOFF"] == 3 and TENSOR["VOFF"] == 4
    lib = _load()
    st = _Store(wl.seed, wl.off_sigma, wl.n_layers, wl.n_kv_heads, wl.block_tokens,
                wl.head_dim, _dtype_code(wl.dtype))
    fn = ctypes.cast(lib.synth_gather_kv, ctypes.c_void_p).value
    return fn, ctypes.addressof(st), st
