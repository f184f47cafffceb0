"""The seeded input generator: compiled form == NumPy restatement, determinism."""
import numpy as np

import synth
from synth import reference as ref


def test_unit_stream_matches_numpy_restatement():
    for (seed, tensor, i0, i1) in [(0, 1, 0, 0), (7, 5, 123, 45), (2**40, 9, 99999, 511)]:
        k = synth.stream_key(seed, tensor, i0, i1)
        assert k == int(ref.key(seed, tensor, i0, i1))
        a = synth.unit_stream(k, 17, 4096)
        b = ref.unit(k, 17, 4096)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_kv_blocks_match_numpy_restatement_bf16_and_f32():
    wl = synth.get_workload("ctx64k")
    got = synth.kv_blocks(wl, "V", 40, 3)
    want = ref.kv_block(wl.seed, 2, 4, 0.5, 42, wl.n_layers, wl.n_kv_heads, 32, wl.head_dim, "bf16")
    assert np.array_equal(got[2], want)
    wt = synth.get_workload("tiny")
    got = synth.kv_blocks(wt, "K", 0, 2)
    want = ref.kv_block(wt.seed, 1, 3, 0.0, 1, 1, 2, 32, 64, "f32")
    assert np.array_equal(got[1].view(np.uint32), want.view(np.uint32))


def test_kv_blocks_match_numpy_restatement_fp8():
    wl = synth.get_workload("ctx64k_fp8")
    got = synth.kv_blocks(wl, "K", 7, 2)
    want = ref.kv_block(wl.seed, 1, 3, 0.5, 8, wl.n_layers, wl.n_kv_heads, 32, wl.head_dim, "fp8")
    assert got.dtype == np.uint8 and np.array_equal(got[1], want)
    # the encoder on its own: ties to even, subnormals, saturation, signed zero
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 463.9, 464.0, 1e6, -0.0, -1e-7,
                  -500.0], dtype=np.float32)
    assert ref.to_e4m3_bits(x).tolist() == [0x38, 0x3A, 0x00, 0x01, 0x7E, 0x7E, 0x7E, 0x80, 0x80,
                                            0xFE]


def test_any_block_regenerates_alone():
    wl = synth.get_workload("ctx64k")
    many = synth.kv_blocks(wl, "K", 100, 8)
    one = synth.kv_blocks(wl, "K", 105, 1)
    assert np.array_equal(many[5], one[0])


def test_query_and_direct_index_match_restatement():
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, n_q_tokens=3)
    q = synth.query(wl)
    k = ref.key(wl.seed, 5, 1, 7)
    want = ref.to_bf16_bits(ref.unit(k, 0, 3 * 128).reshape(3, 128))
    assert np.array_equal(q[1, 7], want)
    w4 = synth.get_workload("ws10m").scaled(n_layers=2)
    idx = synth.index_direct(w4, 1000, 4)
    lg = 1 * 8 + 3
    a = np.float32(0.5) * ref.unit(ref.key(0, 3, 1002, lg), 0, 128)
    c = ref.INV_SQRT32 * ref.unit(ref.key(0, 6, 1002, lg), 0, 128)
    assert np.array_equal(idx[1, 3, 2], ref.to_bf16_bits((a + c).astype(np.float32)))


def test_unit_law_moments():
    x = synth.unit_stream(synth.stream_key(3, 1, 2, 3), 0, 1 << 20).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.var() - 1.0) < 5e-3
    assert np.max(np.abs(x)) <= np.sqrt(3) * 2 + 1e-6


def test_churn_topic_is_deterministic_ar1():
    wl = synth.get_workload("churn").scaled(n_layers=2, n_q_heads=8, n_kv_heads=2)
    u2 = synth.churn_shift(wl, 2)
    assert np.array_equal(u2, synth.churn_shift(wl, 2))
    u1 = synth.churn_shift(wl, 1)
    c = np.corrcoef(u1.ravel(), u2.ravel())[0, 1]
    assert 0.8 < c < 0.97


def test_gather_store_writes_the_generated_block():
    import ctypes
    wl = synth.get_workload("ctx64k").scaled(n_layers=2)
    fn, user, keep = synth.gather_store(wl)
    f = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                         ctypes.c_void_p)(fn)
    for which, name in ((0, "K"), (1, "V")):
        buf = np.empty(wl.block_elems, np.uint16)
        assert f(user, 1234, which, buf.ctypes.data) == 0
        assert np.array_equal(buf, synth.kv_blocks(wl, name, 1234, 1).ravel())
