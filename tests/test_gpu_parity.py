"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Tolerances: Mean-K, selections, compact positions, page tables and V are
bit-exact; scores within 1e-5 relative; re-RoPE'd K within 2e-2 absolute
(bf16) or 1e-5 relative (fp32) of the unrounded float64 oracle.
"""
import numpy as np
import pytest

import synth
from oracle import select_blocks, compact_positions
from oracle.numerics import bf16_bits, fp8_decode, fp8_encode
from oracle import pipeline as op
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def k():
    import torch
    import attention_space_block_amd as kvm
    assert torch.cuda.is_available()
    kvm._abi.lib()
    return kvm


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- Mean-K ----

@pytest.mark.parametrize("name,nb,layers", [("tiny", 128, None), ("ctx64k", 300, 2),
                                             ("ctx64k_fp8", 300, 2)])
def test_build_index_bit_exact(k, dev, name, nb, layers):
    wl = synth.get_workload(name)
    if layers:
        wl = wl.scaled(n_layers=layers)
    say("build_index", name, nb)
    raw = gc.raw_to_device(wl, "K", 0, nb, dev)
    idx = gc.build_index_dev(k, wl, raw, dev)
    want = op.index_rows(wl, 0, nb)
    got = gc.as_f64(gc.to_host_bits(idx))
    assert np.array_equal(got, want)


def test_build_index_append_and_stride(k, dev):
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2)
    raw = gc.raw_to_device(wl, "K", 0, 100, dev)
    full = gc.build_index_dev(k, wl, raw, dev, cap=128)
    part = torch.zeros_like(full)
    dims, dt = k.dims_for(wl), k.KVM_BF16
    k.kvm_build_index(dims, dt, raw, wl.block_bytes, 0, 37, part, 128)
    k.kvm_build_index(dims, dt, raw[37:], wl.block_bytes, 37, 63, part, 128)
    assert torch.equal(full, part)
    # strided source: every other block of a doubled buffer
    dbl = torch.zeros((200, wl.block_elems), dtype=raw.dtype, device=dev)
    dbl[0::2] = raw
    st = torch.zeros_like(full)
    k.kvm_build_index(dims, dt, dbl, 2 * wl.block_bytes, 0, 100, st, 128)
    assert torch.equal(full, st)
    assert int(full[:, :, 100:].abs().sum()) == 0     # rows past the range untouched


# ------------------------------------------- Mean-K from post-RoPE K ----

@pytest.mark.parametrize("name,layout,pos0,N", [
    ("ctx64k", 0, 0, 70), ("ctx64k", 1, 4096, 37), ("tiny", 0, 96, 9), ("tiny", 1, 0, 5),
    ("ctx64k_fp8", 0, 512, 41), ("ctx64k_fp8", 1, 0, 30),
])
def test_build_index_rope_matches_oracle(k, dev, name, layout, pos0, N):
    from oracle import mean_k_from_rope
    wl = synth.get_workload(name).scaled(rope_layout=layout)
    if name.startswith("ctx64k"):
        wl = wl.scaled(n_layers=2)
    idt = wl.index_dtype                                     # bf16 rows for fp8 K
    say("build index rope", name, layout, pos0, N)
    k_rope = synth.kv_blocks(wl, "K", 0, N)                 # any K values stand for cached K
    kd = gc.to_dev(k_rope.reshape(N, -1), dev)
    pool = gc.Pool(k, wl, 4, N, pos0 + 32 * N, dev)
    import torch
    index = torch.zeros((wl.n_layers, wl.n_kv_heads, N + 3, wl.head_dim),
                        dtype=gc.index_torch_dtype(wl), device=dev)
    pool.ctx.kvm_ctx_build_index_rope(kd, wl.block_bytes, 0, N, pos0, index, N + 3)
    got = gc.to_host_bits(index)[:, :, :N]
    kf = op.as_f64(k_rope, wl.dtype)
    want = mean_k_from_rope(kf, pos0, idt, wl.theta, layout)              # [N][L][Hkv][d]
    want = np.transpose(want, (1, 2, 0, 3))
    if idt == "bf16":
        assert np.array_equal(got, bf16_bits(want))
        gv = op.as_f64(got, "bf16")
    else:
        assert np.array_equal(got, want.astype(np.float32))
        gv = got.astype(np.float64)
    exact = np.transpose(mean_k_from_rope(kf, pos0, "f64", wl.theta, layout, table_fp32=False),
                         (1, 2, 0, 3))
    # against the exact float64 rotation: half an ulp of rounding plus the fp32
    # table's error, at most (|a| + |b|) * 2^-24 per pair of a token
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - (7 if idt == "bf16" else 23))
    table_err = 2.0 * np.abs(kf).max() * 2.0 ** -24
    assert np.all(np.abs(gv - exact) <= 0.5 * ulp + table_err)
    assert int(index[:, :, N:].abs().sum()) == 0
    # appending in two calls (positions continue) gives the same rows
    part = torch.zeros_like(index)
    n1 = N // 2
    pool.ctx.kvm_ctx_build_index_rope(kd, wl.block_bytes, 0, n1, pos0, part, N + 3)
    pool.ctx.kvm_ctx_build_index_rope(kd[n1:], wl.block_bytes, n1, N - n1, pos0 + 32 * n1,
                                      part, N + 3)
    assert torch.equal(part, index)
    # positions past the ctx's table are refused
    with pytest.raises(k.KvmError) as e:
        pool.ctx.kvm_ctx_build_index_rope(kd, wl.block_bytes, 0, N, pos0 + 32, index, N + 3)
    assert e.value.code == k.api._abi.KVM_ERANGE
    pool.ctx.close()


# ---------------------------------------------------------------- scores ----

def _score_case(k, dev, wl, N):
    index = op.index_rows(wl, 0, N)
    q = op.query_stored(wl, 0, index)
    ref = op.block_scores(op.as_f64(q, wl.index_dtype), index)
    raw = gc.raw_to_device(wl, "K", 0, N, dev)
    idx_dev = gc.build_index_dev(k, wl, raw, dev)
    got = gc.score_dev(k, wl, gc.to_dev(q, dev), idx_dev, N, N, dev).cpu().numpy()
    return got.astype(np.float64), ref


@pytest.mark.parametrize("name,N,scale", [
    ("tiny", 128, {}),
    ("ctx64k", 2048, {}),                              # MFMA path, full size
    ("ctx64k", 1000, {"n_layers": 2, "n_q_tokens": 77}),  # ragged rows and blocks
    ("ctx64k", 700, {"n_layers": 2, "n_q_tokens": 1}),    # stored path, bf16, d = 128
    ("ctx64k", 333, {"n_layers": 1, "n_q_tokens": 5}),    # stored path, ragged
])
def test_scores_match_oracle(k, dev, name, N, scale):
    wl = synth.get_workload(name).scaled(**scale) if scale else synth.get_workload(name)
    say("scores", name, N, scale)
    got, ref = _score_case(k, dev, wl, N)
    assert abs(got.sum() - wl.n_q_tokens) <= 1e-5 * wl.n_q_tokens
    rel = np.abs(got - ref) / ref
    assert rel.max() <= 1e-5, f"max rel err {rel.max()} at block {rel.argmax()}"


def _e4m3_probe_values(n: int, seed: int) -> np.ndarray:
    """fp32 inputs for the E4M3 conversion: normals over many binades, every
    E4M3 value and every midpoint between neighbours (the ties), values past the
    saturation point, signed zeros, values below half the smallest subnormal,
    and infinities."""
    rng = np.random.default_rng(seed)
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = fp8_decode(codes)
    mids = (vals[1:] + vals[:-1]) / 2
    special = np.r_[vals, -vals, mids, -mids, 448.0, 449.0, 464.0, 480.0, 1e6, -1e6, 0.0, -0.0,
                    2.0 ** -11, -(2.0 ** -11), np.inf, -np.inf]
    rand = rng.standard_normal(n) * np.exp2(rng.integers(-12, 10, n))
    return np.r_[special, rand].astype(np.float32)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_e4m3_bit_exact(k, dev, src):
    """kvm_quantize_e4m3 equals the oracle's E4M3 encoder byte for byte
    (nearest, ties to even, saturating), for a length with a ragged tail."""
    import torch
    x = _e4m3_probe_values(3001, 5)
    if src == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        xin, want = gc.to_dev(bits, dev), fp8_encode(op.as_f64(bits, "bf16"))
        code = k.KVM_BF16
    else:
        xin, want = gc.to_dev(x, dev), fp8_encode(x.astype(np.float64))
        code = k.KVM_F32
    n = x.size
    out = torch.full((n + 5,), 0x5A, dtype=torch.uint8, device=dev)
    k.kvm_quantize_e4m3(xin, code, n, out)
    got = out.cpu().numpy()
    assert np.array_equal(got[:n], want), np.flatnonzero(got[:n] != want)[:10]
    assert np.all(got[n:] == 0x5A)                 # nothing written past n


@pytest.mark.parametrize("N,scale", [
    (1, {"n_layers": 1}),                                         # one block, two-pass form
    (1, {"n_layers": 1, "n_q_tokens": 1}),                        # one block, stored form
    (3, {"n_layers": 1, "n_q_tokens": 11}),                       # T*G = 66 over 3 blocks
    (129, {"n_layers": 1, "n_q_heads": 16, "n_q_tokens": 32}),    # G = 2, T*G = 64: two-pass
    (129, {"n_layers": 1, "n_q_heads": 16, "n_q_tokens": 31}),    # T*G = 62: stored form
    (300, {"n_layers": 1, "n_q_heads": 8, "n_q_tokens": 64}),     # G = 1, T*G = 64
    (300, {"n_layers": 1, "n_q_heads": 8, "n_q_tokens": 63}),     # G = 1, stored form
    (200, {"n_layers": 2, "head_dim": 64, "n_q_tokens": 40}),     # d = 64 bf16, 240 rows
    (1000, {"n_layers": 2, "head_dim": 64, "n_q_tokens": 77}),    # d = 64, 462 ragged rows
    (300, {"n_layers": 2, "head_dim": 64, "n_q_tokens": 5}),      # d = 64, stored form
])
def test_scores_edge_shapes_match_oracle(k, dev, N, scale):
    """Degenerate and boundary shapes: a single block (every softmax is 1, so
    R = T), a handful of blocks on the two-pass form, T*G on either side of
    the 64 rows where the stored-score form takes over, no grouping (G = 1),
    and d = 64 with bf16 on the two-pass (128-byte rows) and stored forms."""
    wl = synth.get_workload("ctx64k").scaled(**scale)
    say("score edge", N, scale)
    got, ref = _score_case(k, dev, wl, N)
    T = wl.n_q_tokens
    assert abs(got.sum() - T) <= 1e-5 * T
    if N == 1:
        assert abs(got[0] - T) <= 1e-5 * T
    rel = np.abs(got - ref) / ref
    assert rel.max() <= 1e-5, f"max rel err {rel.max()} at block {rel.argmax()}"


@pytest.mark.parametrize("N,scale", [
    (2048, {}),                                     # full ctx64k shape
    (1000, {"n_layers": 2, "n_q_tokens": 77}),      # ragged rows (TG 462) and blocks
])
def test_fp8_scores_match_oracle(k, dev, N, scale):
    """FP8 scoring ablation: E4M3 queries and Mean-K (encoded by the oracle) on
    the FP8 matrix-core kernels, against the float64 Eq. (10) of the decoded
    values."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(**scale) if scale else synth.get_workload("ctx64k")
    say("fp8 scores", N, scale)
    index = op.index_rows(wl, 0, N)
    q = op.query_stored(wl, 0, index)
    qb = fp8_encode(op.as_f64(q, "bf16"))
    ib = fp8_encode(index)
    ref = op.block_scores(fp8_decode(qb), fp8_decode(ib))
    dims = k.dims_for(wl)
    T = wl.n_q_tokens
    ws_b = k.kvm_score_ws_bytes(dims, k.KVM_FP8_E4M3, T, N, 0, 0)
    assert ws_b > 0
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    scores = torch.empty(N, dtype=torch.float32, device=dev)
    k.kvm_score_blocks(dims, k.KVM_FP8_E4M3, torch.from_numpy(qb).to(dev), T,
                       torch.from_numpy(np.ascontiguousarray(ib)).to(dev), N, N, 0, 0, scores,
                       ws, ws_b)
    got = scores.cpu().numpy().astype(np.float64)
    assert abs(got.sum() - T) <= 1e-5 * T
    rel = np.abs(got - ref) / ref
    assert rel.max() <= 1e-5, f"max rel err {rel.max()} at block {rel.argmax()}"


@pytest.mark.parametrize("N,T,L", [(700, 1, 2), (333, 5, 1), (1500, 10, 1)])
def test_fp8_stored_scores_match_oracle(k, dev, N, T, L):
    """FP8 scoring ablation on the stored-score path (T*G <= 64: decode-sized
    query rows, 6 to 60 here, ragged against the 16-row tiles and the 512-block
    partials): E4M3 queries and Mean-K against the float64 Eq. (10) of the
    decoded values."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=L, n_q_tokens=T)
    say("fp8 stored scores", N, T, L)
    index = op.index_rows(wl, 0, N)
    q = op.query_stored(wl, 0, index)
    qb = fp8_encode(op.as_f64(q, "bf16"))
    ib = fp8_encode(index)
    ref = op.block_scores(fp8_decode(qb), fp8_decode(ib))
    dims = k.dims_for(wl)
    ws_b = k.kvm_score_ws_bytes(dims, k.KVM_FP8_E4M3, T, N, 0, 0)
    assert ws_b > 0
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    scores = torch.empty(N, dtype=torch.float32, device=dev)
    k.kvm_score_blocks(dims, k.KVM_FP8_E4M3, torch.from_numpy(qb).to(dev), T,
                       torch.from_numpy(np.ascontiguousarray(ib)).to(dev), N, N, 0, 0, scores,
                       ws, ws_b)
    got = scores.cpu().numpy().astype(np.float64)
    assert abs(got.sum() - T) <= 1e-5 * T
    rel = np.abs(got - ref) / ref
    assert rel.max() <= 1e-5, f"max rel err {rel.max()} at block {rel.argmax()}"


def test_fp8_host_tiled_scores_equal_resident(k, dev):
    """An E4M3 index streamed from pinned host memory in 512-block tiles gives
    the same scores, bit for bit, as the same index resident in HBM (same
    kernels, same partial boundaries)."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, n_q_tokens=1)
    N, T, tile = 1300, 1, 512
    say("fp8 host-tiled scores", N)
    index = op.index_rows(wl, 0, N)
    qb = fp8_encode(op.as_f64(op.query_stored(wl, 0, index), "bf16"))
    ib = np.ascontiguousarray(fp8_encode(index))                 # [L][Hkv][N][d]
    dims = k.dims_for(wl)
    q = torch.from_numpy(qb).to(dev)
    ws_r = k.kvm_score_ws_bytes(dims, k.KVM_FP8_E4M3, T, N, 0, 0)
    ws = torch.empty(ws_r, dtype=torch.uint8, device=dev)
    want = torch.empty(N, dtype=torch.float32, device=dev)
    k.kvm_score_blocks(dims, k.KVM_FP8_E4M3, q, T, torch.from_numpy(ib).to(dev), N, N, 0, 0,
                       want, ws, ws_r)
    # host layout: tile-major [tile][L*Hkv][tile_blocks][d], the last tile zero-padded
    nlg, d = wl.n_layers * wl.n_kv_heads, wl.head_dim
    ntile = (N + tile - 1) // tile
    host = torch.zeros(ntile * nlg * tile * d, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy().reshape(ntile, nlg, tile, d)
    flat = ib.reshape(nlg, N, d)
    for t in range(ntile):
        n = min(tile, N - t * tile)
        hv[t, :, :n] = flat[:, t * tile:t * tile + n]
    ws_h = k.kvm_score_ws_bytes(dims, k.KVM_FP8_E4M3, T, N, k.KVM_INDEX_HOST_TILED, tile)
    assert ws_h > 0
    wsh = torch.empty(ws_h, dtype=torch.uint8, device=dev)
    got = torch.empty(N, dtype=torch.float32, device=dev)
    k.kvm_score_blocks(dims, k.KVM_FP8_E4M3, q, T, host, 0, N, k.KVM_INDEX_HOST_TILED, tile,
                       got, wsh, ws_h)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref = op.block_scores(fp8_decode(qb), fp8_decode(ib))
    assert np.max(np.abs(got.cpu().numpy() - ref) / ref) <= 1e-5


def test_fp8_scores_unsupported_forms(k, dev):
    """FP8 scores need d = 128 and either T*G <= 64 or an index in HBM."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=1, n_q_tokens=11)   # T*G = 66 > 64
    dims = k.dims_for(wl)
    assert k.kvm_score_ws_bytes(dims, k.KVM_FP8_E4M3, 11, 256, 0, 0) > 0
    assert k.kvm_score_ws_bytes(dims, k.KVM_FP8_E4M3, 11, 1024, k.KVM_INDEX_HOST_TILED, 512) == 0
    q = torch.zeros(wl.n_layers * wl.n_q_heads * 11 * wl.head_dim, dtype=torch.uint8, device=dev)
    host = torch.zeros(wl.n_layers * wl.n_kv_heads * 1024 * wl.head_dim, dtype=torch.uint8,
                       pin_memory=True)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    scores = torch.empty(1024, dtype=torch.float32, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_score_blocks(dims, k.KVM_FP8_E4M3, q, 11, host, 0, 1024, k.KVM_INDEX_HOST_TILED,
                           512, scores, ws, ws.numel())
    assert e.value.code == k.api._abi.KVM_ENOTSUP


def test_scores_steep_ramp_match_oracle(k, dev):
    """Scores that climb (or fall) by more than 32 log2-units along the block
    axis: rows facing away see most terms vanish, rows facing the ramp put
    their mass on its far end; both must match the float64 softmax. At this
    size pass 1 splits the blocks eight ways, so every workgroup streams 256
    of them and sets its shift on the exact path of its first stage; shift
    refreshes in later stages are the next test's subject."""
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, n_q_tokens=77)
    N, d = 2048, wl.head_dim
    import torch
    noise = op.as_f64(synth.index_direct(wl, 0, N), "bf16")       # [L][Hkv][N][d]
    ramp = np.linspace(-120.0, 120.0, N)[None, None, :, None] / np.sqrt(d)
    bits = torch.from_numpy((noise + ramp).astype(np.float32)).to(torch.bfloat16)
    bits = bits.view(torch.int16).numpy().view(np.uint16)          # the input, as bf16
    q = synth.query(wl)
    ref = op.block_scores(op.as_f64(q, "bf16"), op.as_f64(bits, "bf16"))
    got = gc.score_dev(k, wl, gc.to_dev(q, dev), gc.to_dev(bits, dev), N, N,
                       dev).cpu().numpy().astype(np.float64)
    assert abs(got.sum() - wl.n_q_tokens) <= 1e-5 * wl.n_q_tokens
    # the input does what it is for: a third of the query rows see their scores
    # span more than 32 log2-units across the blocks (magnitudes stay below 64,
    # where fp32 exp arguments keep the 1e-5 bound)
    qf = op.as_f64(q, "bf16").reshape(wl.n_layers, wl.n_kv_heads, -1, d)
    kf = op.as_f64(bits, "bf16")
    span = np.stack([np.ptp(qf[l, g] @ kf[l, g].T, axis=1) for l in range(wl.n_layers)
                     for g in range(wl.n_kv_heads)]) * np.log2(np.e) / np.sqrt(d)
    assert np.mean(span > 32) > 0.25
    assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-30)


@pytest.mark.parametrize("shape,d", [("step", 128), ("linear", 128), ("step", 64)])
def test_scores_shift_refresh_after_first_stage(k, dev, shape, d):
    """Scores that rise by more than 64 log2-units after a workgroup's first
    stage: pass 1 sums each stage's exps against the shift it started with and
    takes the stage again exactly when a sum passes 2^64, so these rows must
    refresh their shift in a later stage. 512 (layer, KV head) pairs x 4 row
    chunks keep every workgroup on the whole block range (one split), so the
    rise falls inside one workgroup's stream. Coordinate 0 of the index carries
    the rise (+-R along the blocks) and coordinate 0 of the queries is +-4, so
    half of the rows climb and half fall by 70-80 log2-units, with scores
    below 50 in magnitude. "step": one jump at block 900, inside the ragged
    last stage (blocks 896..935), whose re-take also covers a partly valid and
    an empty subtile; "linear": a ramp across all 936 blocks; d = 64 runs the
    128-byte-row form. The FP8 form of the kernel takes the same re-take code
    (its first-stage re-takes run in every FP8 scoring test), but its matrix
    instruction sums each 64-long dot product to only about 11-13 bits below
    the largest product, which at these score magnitudes (products near 290)
    puts single scores outside 1e-5, so it is left out here."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=64, n_q_tokens=160, head_dim=d)
    N = 936
    say("shift refresh", shape, d, N)
    scale = np.log2(np.e) / np.sqrt(d)
    # the same rise in log2 units at d = 64 as at d = 128
    R = (70.0 if shape == "step" else 80.0) * (np.log2(np.e) / np.sqrt(128)) / scale
    ramp = (np.where(np.arange(N) >= 900, R, -R) if shape == "step"
            else np.linspace(-R, R, N))
    ix = op.as_f64(synth.index_direct(wl, 0, N), "bf16")         # [L][Hkv][N][d]
    ix[:, :, :, 0] += ramp[None, None, :]
    qf = op.as_f64(synth.query(wl), "bf16")                       # [L][Hq][T][d]
    qf[:, :, :, 0] = np.where(np.arange(wl.n_q_tokens) % 2 == 0, 4.0, -4.0)[None, None, :]
    ib = torch.from_numpy(ix.astype(np.float32)).to(torch.bfloat16)
    ib = ib.view(torch.int16).numpy().view(np.uint16)
    qb = torch.from_numpy(qf.astype(np.float32)).to(torch.bfloat16)
    qb = qb.view(torch.int16).numpy().view(np.uint16)
    kf, qf = op.as_f64(ib, "bf16"), op.as_f64(qb, "bf16")
    # the input does what it is for (layer 0): every climbing row ends more
    # than 64 log2-units above the largest score of blocks 0..95 (the first
    # stage's exps), and no score reaches 64 in magnitude
    G = wl.n_q_heads // wl.n_kv_heads
    for g in range(wl.n_kv_heads):
        x = qf[0, g * G:(g + 1) * G].reshape(-1, d) @ kf[0, g].T * scale
        up = x[np.tile(np.arange(wl.n_q_tokens) % 2 == 0, G)]
        assert np.all(up.max(axis=1) - up[:, :96].max(axis=1) > 66)
        assert np.abs(x).max() < 64
    ref = op.block_scores(qf, kf)
    scores = gc.score_dev(k, wl, gc.to_dev(qb, dev), gc.to_dev(ib, dev), N, N, dev)
    got = scores.cpu().numpy().astype(np.float64)
    assert abs(got.sum() - wl.n_q_tokens) <= 1e-5 * wl.n_q_tokens
    assert np.all(np.abs(got - ref) <= 1e-5 * ref + 1e-30)


def test_host_tiled_scores_equal_resident(k, dev):
    import torch
    wl = synth.get_workload("ws10m").scaled(n_layers=4, n_blocks=1300, tile_blocks=512)
    N, tb, nlg, d = wl.n_blocks, wl.tile_blocks, wl.n_layers * wl.n_kv_heads, wl.head_dim
    say("host tiled", N, tb)
    ntile = (N + tb - 1) // tb
    index = synth.index_direct(wl, 0, N)                      # [L][Hkv][N][d]
    host = torch.zeros((ntile, nlg, tb, d), dtype=torch.int16).pin_memory()
    hv = host.numpy().view(np.uint16)
    ix = index.reshape(nlg, N, d)
    for t in range(ntile):
        n = min(tb, N - t * tb)
        hv[t, :, :n] = ix[:, t * tb:t * tb + n]
    q = synth.query(wl)
    qd = gc.to_dev(q, dev)
    idx_dev = gc.to_dev(index, dev)
    res = gc.score_dev(k, wl, qd, idx_dev, N, N, dev).cpu().numpy()
    til = gc.score_dev(k, wl, qd, None, N, N, dev, loc=1, tile_blocks=tb,
                       host_index=host).cpu().numpy()
    assert np.array_equal(res, til)
    ref = op.block_scores(op.as_f64(q, "bf16"), op.as_f64(index, "bf16"))
    assert np.max(np.abs(res - ref) / ref) <= 1e-5


def test_host_tiled_wide_query_rows_match_oracle(k, dev):
    """72 query rows per (l, g) from a host-tiled index: the stored-score path
    with more rows than its matrix-core kernel takes (the VALU kernel and the
    separate stats pass), against the oracle."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, n_q_tokens=12)
    N, tb, nlg, d = 1300, 512, wl.n_layers * wl.n_kv_heads, wl.head_dim
    ntile = (N + tb - 1) // tb
    index = synth.index_direct(wl.scaled(index_direct=True), 0, N)
    host = torch.zeros((ntile, nlg, tb, d), dtype=torch.int16).pin_memory()
    hv = host.numpy().view(np.uint16)
    ix = index.reshape(nlg, N, d)
    for t in range(ntile):
        n = min(tb, N - t * tb)
        hv[t, :, :n] = ix[:, t * tb:t * tb + n]
    q = synth.query(wl)
    til = gc.score_dev(k, wl, gc.to_dev(q, dev), None, N, N, dev, loc=1, tile_blocks=tb,
                       host_index=host).cpu().numpy().astype(np.float64)
    ref = op.block_scores(op.as_f64(q, "bf16"), op.as_f64(index, "bf16"))
    assert np.max(np.abs(til - ref) / ref) <= 1e-5


# ---------------------------------------------------------------- select ----

@pytest.mark.parametrize("N,sink,recent,budget,kind", [
    (128, 1, 2, 11, "cont"), (2048, 1, 64, 512, "ties"), (32768, 1, 64, 4096, "cont"),
    (32768, 1, 64, 4096, "ties"), (312500, 1, 256, 2048, "cont"), (5000, 0, 0, 100, "const"),
    (600, 3, 5, 8, "ties"), (500, 1, 64, 512, "cont"), (512, 1, 64, 512, "ties"), (1, 1, 0, 1, "cont"),
])
def test_select_bit_exact(k, dev, N, sink, recent, budget, kind):
    say("select", N, sink, recent, budget, kind)
    R = synth.scores_f32(N + budget, N, kind=kind, levels=4)
    sel, n_sel, base = gc.select_dev(k, gc.to_dev(R, dev), N, sink, recent, budget, dev)
    want = select_blocks(R, sink, recent, budget)
    n = int(n_sel.item())
    assert n == len(want) == min(N, budget)
    assert np.array_equal(sel.cpu().numpy()[:n], want)
    assert np.array_equal(base.cpu().numpy()[:n], compact_positions(n))


def test_select_error_paths(k, dev):
    R = synth.scores_f32(9, 1000)
    for bad in (np.nan, -1.0, np.inf):
        R2 = R.copy()
        R2[500] = bad
        _, n_sel, _ = gc.select_dev(k, gc.to_dev(R2, dev), 1000, 1, 8, 100, dev)
        assert int(n_sel.item()) == k.api._abi.KVM_ERANGE
    with pytest.raises(k.KvmError) as e:
        gc.select_dev(k, gc.to_dev(R, dev), 1000, 60, 60, 100, dev)
    assert e.value.code == k.api._abi.KVM_ERANGE
    # a bad score in the sink, the recent region and the last (partial) chunk
    R = synth.scores_f32(10, 9000)
    for pos in (0, 8999, 8192, 4096):
        R2 = R.copy()
        R2[pos] = np.nan
        _, n_sel, _ = gc.select_dev(k, gc.to_dev(R2, dev), 9000, 1, 8, 100, dev)
        assert int(n_sel.item()) == k.api._abi.KVM_ERANGE
    # a workspace smaller than kvm_select_ws_bytes
    import torch
    sel = torch.empty(100, dtype=torch.int32, device=dev)
    n_sel = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(k.kvm_select_ws_bytes(9000) - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_select(gc.to_dev(R, dev), 9000, 1, 8, 100, 32, sel, n_sel, sel, ws, ws.numel())
    assert e.value.code == k.api._abi.KVM_ENOMEM


@pytest.mark.parametrize("N,sink,recent,budget,kind", [
    (5000, 50, 50, 100, "cont"),        # no free slots: sink and recent only
    (20000, 1, 3, 5000, "const"),       # every candidate ties, across chunk boundaries
    (8192, 0, 0, 4097, "ties"),         # chunk-aligned N
    (8193, 2, 0, 4096, "ties"),         # one block in the last chunk
    (12287, 0, 7, 3000, "cont"),
])
def test_select_chunked_cases(k, dev, N, sink, recent, budget, kind):
    say("select chunked", N, sink, recent, budget, kind)
    R = synth.scores_f32(N + 3 * budget, N, kind=kind, levels=3)
    sel, n_sel, base = gc.select_dev(k, gc.to_dev(R, dev), N, sink, recent, budget, dev)
    want = select_blocks(R, sink, recent, budget)
    n = int(n_sel.item())
    assert n == len(want) == budget
    assert np.array_equal(sel.cpu().numpy()[:n], want)
    assert np.array_equal(base.cpu().numpy()[:n], compact_positions(n))


def test_select_signed_zero_and_subnormal(k, dev):
    """-0.0 equals 0.0 (a tie, lower id first); positive subnormals rank above
    zero and below every normal number."""
    N = 10000
    R = np.zeros(N, dtype=np.float32)
    R[1::3] = -0.0
    tiny = np.float32(1e-44)                       # subnormal
    R[5::97] = tiny
    R[7::89] = np.float32(2.0) * tiny
    R[11::1009] = np.float32(1e-3)
    for budget in (40, 150, 300):
        sel, n_sel, _ = gc.select_dev(k, gc.to_dev(R, dev), N, 1, 2, budget, dev)
        want = select_blocks(R, 1, 2, budget)
        n = int(n_sel.item())
        assert n == budget
        assert np.array_equal(sel.cpu().numpy()[:n], want)


def test_select_workspace_reuse(k, dev):
    """Two selections in a row on one workspace: the second starts from reset
    control words."""
    import torch
    N, budget = 50000, 2048
    ws = torch.empty(k.kvm_select_ws_bytes(N), dtype=torch.uint8, device=dev)
    sel = torch.empty(budget, dtype=torch.int32, device=dev)
    n_sel = torch.empty(1, dtype=torch.int32, device=dev)
    base = torch.empty(budget, dtype=torch.int32, device=dev)
    for seed, kind, n in ((21, "ties", N), (22, "cont", N - 4096)):
        R = synth.scores_f32(seed, n, kind=kind, levels=5)
        k.kvm_select(gc.to_dev(R, dev), n, 1, 64, budget, 32, sel, n_sel, base, ws, ws.numel())
        want = select_blocks(R, 1, 64, budget)
        assert int(n_sel.item()) == budget
        assert np.array_equal(sel.cpu().numpy()[:budget], want)


# ------------------------------------------------------ rematerialization ----

def _remat_setup(k, dev, wl, N, n_slots, src="device", batch=64, staging=0, delta_limit=0,
                 max_pos=None):
    import torch
    pool = gc.Pool(k, wl, n_slots, N, max_pos or wl.budget_blocks * wl.block_tokens, dev, batch,
                   staging, delta_limit)
    keep = []
    if src == "device":
        rk = gc.raw_to_device(wl, "K", 0, N, dev)
        rv = gc.raw_to_device(wl, "V", 0, N, dev)
        pool.ctx.kvm_ctx_set_source(0, N, rk, rv, wl.block_bytes, k.KVM_SRC_DEVICE)
        keep += [rk, rv]
    elif src == "pinned":
        rk = torch.empty((N, wl.block_elems), dtype=gc.torch_dtype(wl)).pin_memory()
        rv = torch.empty((N, wl.block_elems), dtype=gc.torch_dtype(wl)).pin_memory()
        synth.kv_blocks(wl, "K", 0, N, out=rk.numpy().view(gc.np_elem(wl)))
        synth.kv_blocks(wl, "V", 0, N, out=rv.numpy().view(gc.np_elem(wl)))
        pool.ctx.kvm_ctx_set_source(0, N, rk, rv, wl.block_bytes, k.KVM_SRC_HOST_PINNED)
        keep += [rk, rv]
    else:
        import ctypes

        def gather(block, which, dst):
            buf = (ctypes.c_char * wl.block_bytes).from_address(dst)
            arr = np.frombuffer(buf, dtype=gc.np_elem(wl))
            synth.kv_blocks(wl, "K" if which == 0 else "V", block, 1, out=arr, nthreads=1)
            return 0
        pool.ctx.kvm_ctx_set_gather(0, N, gather)
    return pool, keep


@pytest.mark.parametrize("src,delta", [("pinned", 0), ("gather", 0), ("pinned", 2)])
def test_serialized_copies_give_identical_views(k, dev, src, delta):
    """Race check (KVMem Fig. 3: staged copies overlap the re-encode): three
    rematerializations (all misses; about half of the view kept; half of that
    kept again) on two fresh pools, one with the H2D batches on the side
    streams and one with every copy on the caller's stream
    (kvm_ctx_set_serialized). Stats, page tables and every K and V page of the
    views agree byte for byte; without delta mode the serialized views also
    match the oracle."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, budget_blocks=96, n_recent=8)
    N, B = 400, wl.block_tokens
    say("serialized vs overlapped", src, delta)
    sels = []
    keep_from = None
    for t in range(3):
        R = synth.scores_f32(31 + t, N)
        if keep_from is not None:
            R[keep_from] += 10.0
        sel, n_sel, _ = gc.select_dev(k, gc.to_dev(R, dev), N, wl.n_sink, wl.n_recent,
                                      wl.budget_blocks, dev)
        s = sel.cpu().numpy()[:int(n_sel.item())]
        sels.append((sel, n_sel, s))
        keep_from = s[t % 2::2]
    runs = []
    for serialized in (False, True):
        pool, keep = _remat_setup(k, dev, wl, N, 130, src, batch=16, staging=32,
                                  delta_limit=delta, max_pos=N * B)
        pool.ctx.kvm_ctx_set_serialized(serialized)
        out = []
        for sel, n_sel, s in sels:
            st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
            torch.cuda.synchronize()
            pg = pool.page.cpu().numpy()[:len(s)].copy()
            idx = torch.as_tensor(pg.astype(np.int64), device=dev)
            out.append((st, pg, pool.k_view[idx].cpu().numpy(), pool.v_view[idx].cpu().numpy()))
        if serialized and delta == 0:
            gc.check_view(wl, sels[-1][2], out[-1][1], pool)
        pool.ctx.close()
        runs.append(out)
    for t, (a, b) in enumerate(zip(*runs)):
        assert a[0] == b[0], (t, a[0], b[0])
        assert np.array_equal(a[1], b[1]), t
        assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3]), t
    assert runs[0][1][0]["hits"] > 0 and runs[0][2][0]["misses"] > 0


@pytest.mark.parametrize("name,src", [("ctx64k", "device"), ("ctx64k", "pinned"),
                                      ("ctx64k", "gather"), ("ctx64k_fp8", "device"),
                                      ("ctx64k_fp8", "pinned"), ("ctx64k_fp8", "gather")])
def test_remat_view_matches_oracle(k, dev, name, src):
    wl = synth.get_workload(name).scaled(n_layers=2, budget_blocks=96, n_recent=8)
    say("remat", name, src)
    _remat_two_steps(k, dev, wl, src)


def test_fp32_head_dim_128_build_and_remat_match_oracle(k, dev):
    """fp32 K/V at d = 128 (interleaved pairs): Mean-K bit-exact, then the two
    rematerialization steps."""
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, dtype="f32")
    raw = gc.raw_to_device(wl, "K", 0, 130, dev)
    idx = gc.build_index_dev(k, wl, raw, dev)
    assert np.array_equal(gc.as_f64(gc.to_host_bits(idx)), op.index_rows(wl, 0, 130))
    _remat_two_steps(k, dev, wl.scaled(budget_blocks=96, n_recent=8), "pinned")


@pytest.mark.parametrize("name", ["ctx64k", "ctx64k_fp8"])
def test_head_dim_64_build_and_remat_match_oracle(k, dev, name):
    """d = 64 with interleaved pairs, bf16 and FP8 K: the Mean-K rows bit-exact
    against the oracle, then the two rematerialization steps."""
    wl = synth.get_workload(name).scaled(n_layers=2, head_dim=64)
    say("d = 64", name)
    raw = gc.raw_to_device(wl, "K", 0, 130, dev)
    idx = gc.build_index_dev(k, wl, raw, dev)
    assert np.array_equal(gc.as_f64(gc.to_host_bits(idx)), op.index_rows(wl, 0, 130))
    _remat_two_steps(k, dev, wl.scaled(budget_blocks=96, n_recent=8), "device")


@pytest.mark.parametrize("name,scale,src", [
    ("ctx64k", {}, "device"), ("ctx64k_fp8", {}, "gather"), ("tiny", {}, "device"),
    ("ctx64k", {"head_dim": 64}, "pinned"), ("ctx64k_fp8", {"head_dim": 64}, "device"),
    ("ctx64k", {"dtype": "f32"}, "device"),
])
def test_remat_half_split_pairs_match_oracle(k, dev, name, scale, src):
    """The same two steps with RoPE's half-split pairing (t, t + d/2): bf16,
    FP8 and fp32 pages, d = 128 and 64."""
    wl = synth.get_workload(name).scaled(n_layers=2, budget_blocks=96, n_recent=8,
                                         rope_layout=1, **scale)
    say("remat half-split", name, scale, src)
    _remat_two_steps(k, dev, wl, src)


@pytest.mark.parametrize("layout,src", [(0, "device"), (1, "pinned"), (0, "gather")])
def test_fp8_remat_partial_unit_groups_match_oracle(k, dev, layout, src):
    """FP8 pages with 3 layers x 2 KV heads = 6 (layer, KV head) units: an FP8
    work item rotates its piece in several units per (cos, sin) read, so its
    last group here holds fewer units than the others. The two
    rematerialization steps against the oracle, both pairings."""
    wl = synth.get_workload("ctx64k_fp8").scaled(n_layers=3, n_kv_heads=2, n_q_heads=4,
                                                 budget_blocks=96, n_recent=8,
                                                 rope_layout=layout)
    say("fp8 partial unit groups", layout, src)
    _remat_two_steps(k, dev, wl, src)


def _remat_two_steps(k, dev, wl, src):
    """Two rematerializations of a 96-block view over 130 pages: all misses,
    then a selection that keeps about half of the view (hits stay in place,
    their positions change); every page against the oracle."""
    N = 400
    pool, keep = _remat_setup(k, dev, wl, N, 130, src, batch=16, staging=32)
    R = synth.scores_f32(21, N)
    sel, n_sel, base = gc.select_dev(k, gc.to_dev(R, dev), N, wl.n_sink, wl.n_recent,
                                     wl.budget_blocks, dev)
    st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    import torch
    torch.cuda.synchronize()
    n = int(n_sel.item())
    s = sel.cpu().numpy()[:n]
    pg = pool.page.cpu().numpy()[:n]
    assert st["n_sel"] == n == 96 and st["misses"] == 96 and st["hits"] == 0
    assert len(set(pg.tolist())) == n and pg.min() >= 0 and pg.max() < 130
    gc.check_view(wl, s, pg, pool)
    # next step: a shifted selection; hits keep their pages, positions change
    R2 = synth.scores_f32(22, N)
    R2[s[::2]] += 10.0                       # keep about half of the old view
    sel2, n_sel2, _ = gc.select_dev(k, gc.to_dev(R2, dev), N, wl.n_sink, wl.n_recent,
                                    wl.budget_blocks, dev)
    st2 = pool.ctx.kvm_rematerialize(sel2, n_sel2, pool.page)
    torch.cuda.synchronize()
    s2 = sel2.cpu().numpy()[:n]
    pg2 = pool.page.cpu().numpy()[:n]
    old = dict(zip(s.tolist(), pg.tolist()))
    hits = [b for b in s2.tolist() if b in old]
    assert st2["hits"] == len(hits) and st2["misses"] == n - len(hits)
    for b, p in zip(s2.tolist(), pg2.tolist()):
        if b in old:
            assert p == old[b]               # GPU hits reuse their page in place
    assert len(set(pg2.tolist())) == n
    gc.check_view(wl, s2, pg2, pool)
    pool.ctx.close()


@pytest.mark.parametrize("src,layout", [("device", 0), ("pinned", 0), ("gather", 0),
                                        ("device", 1)])
def test_delta_rerope_bounded_and_rebuilt(k, dev, src, layout):
    """Bounded delta re-RoPE (limit 2): three tracked blocks keep being selected
    while the number of earlier blocks in the view changes, so their compact
    positions shift; every third change rebuilds K from raw K."""
    import torch
    from oracle import bounded_delta_rope, rope_rotate
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, rope_layout=layout)
    N, B, limit = 64, wl.block_tokens, 2
    pool, keep = _remat_setup(k, dev, wl, N, 40, src, batch=4, staging=8, delta_limit=limit,
                              max_pos=N * B)
    assert pool.k_shadow is None
    tracked = [30, 31, 45]
    prefix = [5, 9, 2, 12, 12, 7, 3, 10]
    placements = {}                                   # block -> base positions when selected
    raw_k = {b: op.as_f64(synth.kv_blocks(wl, "K", b, 1)[0], "bf16") for b in range(N)}
    for t, a in enumerate(prefix):
        sel_list = list(range(a)) + tracked
        for i, b in enumerate(sel_list):
            placements.setdefault(b, []).append(i * B)
        sel = torch.tensor(sel_list, dtype=torch.int32, device=dev)
        n_sel = torch.tensor([len(sel_list)], dtype=torch.int32, device=dev)
        st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
        torch.cuda.synchronize()
        pg = pool.page.cpu().numpy()[:len(sel_list)]
        kinds_now, worst = {}, 0.0
        for i, b in enumerate(sel_list):
            xs, kinds, counts = bounded_delta_rope(raw_k[b], placements[b], limit, "bf16",
                                                   layout=wl.rope_layout)
            kinds_now[b] = kinds[-1]
            assert pool.ctx.kvm_ctx_block_deltas(b) == counts[-1]
            got = op.as_f64(gc.to_host_bits(pool.k_view[int(pg[i])]).reshape(raw_k[b].shape),
                            "bf16")
            exact = rope_rotate(raw_k[b], i * B + np.arange(B), layout=wl.rope_layout)
            worst = max(worst, gc.pair_error_in_bound(got, exact, counts[-1], wl.rope_layout))
            if kinds[-1] == "full":
                assert np.max(np.abs(got - exact)) <= 2e-2
            v = gc.to_host_bits(pool.v_view[int(pg[i])])
            assert np.array_equal(v, synth.kv_blocks(wl, "V", b, 1).reshape(-1))
        want = {kd: sum(1 for x in kinds_now.values() if x == kd) for kd in ("delta", "full")}
        misses = sum(1 for b in sel_list if len(placements[b]) == 1)
        assert st["misses"] == misses and st["deltas"] == want["delta"]
        assert st["rebuilds"] == want["full"] - misses
        say(f"step {t}: prefix {a}, deltas {st['deltas']}, rebuilds {st['rebuilds']}, "
            f"misses {st['misses']}, worst pair error {worst:.2f} ulp")
    kinds_30 = bounded_delta_rope(raw_k[30], placements[30], limit, "bf16",
                                  layout=wl.rope_layout)[1]
    assert kinds_30 == ["full", "delta", "delta", "full", "same", "delta", "delta", "full"]
    pool.ctx.close()


@pytest.mark.parametrize("scale", [
    {"n_layers": 2},
    {"n_layers": 3, "n_kv_heads": 2, "n_q_heads": 4},   # 6 units: a partial unit group
])
def test_delta_rerope_fp8_pages_bounded(k, dev, scale):
    """Bounded delta re-RoPE over FP8 E4M3 pages (limit 2): the same tracked
    placements as the bf16 test. Each in-place rotation decodes E4M3 exactly,
    rotates in fp32 and stores one E4M3 value, so a pair's error after n deltas
    stays within (n + 1) half-spacings of E4M3 at the pair's length (subnormal
    spacing 2^-9 below 2^-6), plus the fp32 rotation's error; rebuilds from raw
    K are within half a spacing of the exact value. V stays byte-exact. The
    second shape has 6 (layer, KV head) units, not a multiple of the units an
    FP8 work item rotates per table read."""
    import torch
    from oracle import bounded_delta_rope, rope_rotate
    wl = synth.get_workload("ctx64k_fp8").scaled(**scale)
    say("fp8 delta", scale)
    N, B, limit = 64, wl.block_tokens, 2
    pool, keep = _remat_setup(k, dev, wl, N, 40, "device", batch=4, staging=8,
                              delta_limit=limit, max_pos=N * B)
    tracked = [30, 31, 45]
    prefix = [5, 9, 2, 12, 12, 7, 3, 10]
    placements = {}
    raw_k = {b: fp8_decode(synth.kv_blocks(wl, "K", b, 1)[0]) for b in range(N)}
    for t, a in enumerate(prefix):
        sel_list = list(range(a)) + tracked
        for i, b in enumerate(sel_list):
            placements.setdefault(b, []).append(i * B)
        sel = torch.tensor(sel_list, dtype=torch.int32, device=dev)
        n_sel = torch.tensor([len(sel_list)], dtype=torch.int32, device=dev)
        st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
        torch.cuda.synchronize()
        pg = pool.page.cpu().numpy()[:len(sel_list)]
        for i, b in enumerate(sel_list):
            _, kinds, counts = bounded_delta_rope(raw_k[b], placements[b], limit, "fp8")
            assert pool.ctx.kvm_ctx_block_deltas(b) == counts[-1]
            got = fp8_decode(pool.k_view[int(pg[i])].cpu().numpy()).reshape(raw_k[b].shape)
            exact = rope_rotate(raw_k[b], i * B + np.arange(B))
            ea, eb = got[..., 0::2] - exact[..., 0::2], got[..., 1::2] - exact[..., 1::2]
            err = np.hypot(ea, eb)
            norm = np.hypot(exact[..., 0::2], exact[..., 1::2])
            grown = norm * (1 + 0.1 * (counts[-1] + 1))          # length after rounding
            spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(grown, 2.0 ** -100))) - 3),
                                 2.0 ** -9)
            bound = (counts[-1] + 1) * (np.sqrt(2) / 2 * spacing) + 1e-6 * norm
            assert np.all(err <= bound), f"block {b} after {counts[-1]} deltas"
            v = pool.v_view[int(pg[i])].cpu().numpy()
            assert np.array_equal(v, synth.kv_blocks(wl, "V", b, 1).reshape(-1))
        say(f"fp8 step {t}: prefix {a}, deltas {st['deltas']}, rebuilds {st['rebuilds']}, "
            f"misses {st['misses']}")
    kinds_30 = bounded_delta_rope(raw_k[30], placements[30], limit, "fp8")[1]
    assert kinds_30 == ["full", "delta", "delta", "full", "same", "delta", "delta", "full"]
    pool.ctx.close()


def test_delta_rerope_error_growth(k, dev):
    """One block shifted 12 times with a limit of 12: the K error after n
    deltas stays within (n + 1) * sqrt(2)/2 ulp per pair; the printed worst
    errors show how it grows with the count."""
    import torch
    from oracle import rope_rotate
    wl = synth.get_workload("ctx64k").scaled(n_layers=2)
    N, B = 40, wl.block_tokens
    pool, keep = _remat_setup(k, dev, wl, N, 48, "device", delta_limit=12, max_pos=N * B)
    raw = op.as_f64(synth.kv_blocks(wl, "K", 39, 1)[0], "bf16")
    growth = []
    for t, a in enumerate([0, 17, 3, 29, 8, 22, 1, 33, 12, 27, 5, 38, 14]):
        sel_list = list(range(a)) + [39]
        sel = torch.tensor(sel_list, dtype=torch.int32, device=dev)
        n_sel = torch.tensor([len(sel_list)], dtype=torch.int32, device=dev)
        pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
        torch.cuda.synchronize()
        slot = int(pool.page.cpu().numpy()[len(sel_list) - 1])
        got = op.as_f64(gc.to_host_bits(pool.k_view[slot]).reshape(raw.shape), "bf16")
        exact = rope_rotate(raw, a * B + np.arange(B))
        n = pool.ctx.kvm_ctx_block_deltas(39)
        assert n == t
        growth.append((n, gc.pair_error_in_bound(got, exact, n, wl.rope_layout),
                       float(np.max(np.abs(got - exact)))))
    say("delta count, worst pair error (ulp of the pair length), worst abs error:")
    for n, e_ulp, e_abs in growth:
        say(f"  {n:2d}  {e_ulp:5.2f}  {e_abs:.4f}")
    pool.ctx.close()


def test_remat_unchanged_position_is_not_rewritten(k, dev):
    import torch
    wl = synth.get_workload("tiny")
    pool, keep = _remat_setup(k, dev, wl, 128, 16)
    sel = torch.tensor(list(range(11)), dtype=torch.int32, device=dev)
    n_sel = torch.tensor([11], dtype=torch.int32, device=dev)
    st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    st2 = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    assert st["rotated"] == 11 and st2["rotated"] == 0 and st2["hits"] == 11
    torch.cuda.synchronize()
    gc.check_view(wl, sel.cpu().numpy(), pool.page.cpu().numpy()[:11], pool)


def test_memory_range_checks(k, dev):
    """Pointer arguments are checked against their allocation before any work
    is queued: ranges past the end of an allocation, pageable host memory and
    device memory where pinned host memory is required are KVM_EINVAL. The cases
    are chosen so that nothing would be touched out of bounds even without the
    checks (one (layer, KV head), so only in-range rows are ever read)."""
    import torch
    EINVAL = k.api._abi.KVM_EINVAL
    dims = k.Dims(1, 1, 6, 128, 32)
    page = 32 * 128 * 2
    huge = 1 << 28                                   # rows claimed: 64 GiB of index
    # an index capacity far beyond the allocation
    q = torch.zeros(6 * 16 * 128, dtype=torch.int16, device=dev)
    index = torch.zeros(256 * 128, dtype=torch.int16, device=dev)
    ws_b = k.kvm_score_ws_bytes(dims, k.KVM_BF16, 16, 256, 0, 0)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    scores = torch.empty(256, dtype=torch.float32, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_score_blocks(dims, k.KVM_BF16, q, 16, index, huge, 256, 0, 0, scores, ws, ws_b)
    assert e.value.code == EINVAL and "past the end" in str(e.value)
    raw = torch.zeros(4 * page // 2, dtype=torch.int16, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_build_index(dims, k.KVM_BF16, raw, page, 0, 4, index, huge)
    assert e.value.code == EINVAL and "past the end" in str(e.value)
    # a host-tiled index must be pinned host memory
    ws_t = k.kvm_score_ws_bytes(dims, k.KVM_BF16, 1, 512, k.KVM_INDEX_HOST_TILED, 512)
    wst = torch.empty(ws_t, dtype=torch.uint8, device=dev)
    dev_tiles = torch.zeros(512 * 128, dtype=torch.int16, device=dev)
    s512 = torch.empty(512, dtype=torch.float32, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_score_blocks(dims, k.KVM_BF16, q, 1, dev_tiles, 0, 512, k.KVM_INDEX_HOST_TILED,
                           512, s512, wst, ws_t)
    assert e.value.code == EINVAL and "pinned host" in str(e.value)
    # lower-tier sources: kind and residency
    pool = [torch.zeros((4, page // 2), dtype=torch.int16, device=dev) for _ in range(3)]
    ctx = k.KvmCtx(dims, k.KVM_BF16, pool[0], pool[1], pool[2], 4, 16, 4096)
    src_dev = torch.zeros((2, page // 2), dtype=torch.int16, device=dev)
    src_cpu = torch.zeros((2, page // 2), dtype=torch.int16)
    src_pin = torch.zeros((2, page // 2), dtype=torch.int16).pin_memory()
    with pytest.raises(k.KvmError) as e:
        ctx.kvm_ctx_set_source(0, 2, src_dev, src_dev, page, k.KVM_SRC_HOST_PINNED)
    assert e.value.code == EINVAL and "pinned host" in str(e.value)
    with pytest.raises(k.KvmError) as e:
        ctx.kvm_ctx_set_source(0, 2, src_cpu, src_cpu, page, k.KVM_SRC_DEVICE)
    assert e.value.code == EINVAL and "not in memory allocated through HIP" in str(e.value)
    with pytest.raises(k.KvmError) as e:                 # 3 blocks from a 2-block buffer
        ctx.kvm_ctx_set_source(0, 3, src_pin, src_pin, page, k.KVM_SRC_HOST_PINNED)
    assert e.value.code == EINVAL
    ctx.kvm_ctx_set_source(0, 2, src_pin, src_pin, page, k.KVM_SRC_HOST_PINNED)
    ctx.kvm_ctx_set_source(0, 2, src_dev, src_dev, page, k.KVM_SRC_DEVICE)
    ctx.close()
    # a pool in pageable memory
    cpu_pool = torch.zeros((4, page // 2), dtype=torch.int16)
    with pytest.raises(k.KvmError) as e:
        k.KvmCtx(dims, k.KVM_BF16, cpu_pool, cpu_pool, cpu_pool, 4, 16, 4096)
    assert e.value.code == EINVAL
    torch.cuda.synchronize()


def test_remat_error_paths(k, dev):
    import torch
    wl = synth.get_workload("tiny")
    pool = gc.Pool(k, wl, 8, 128, 11 * 32, dev)
    sel = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    n_sel = torch.tensor([3], dtype=torch.int32, device=dev)
    with pytest.raises(k.KvmError) as e:          # no source recorded
        pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    assert e.value.code == k.api._abi.KVM_ERANGE
    n_sel.fill_(9)
    with pytest.raises(k.KvmError) as e:          # view larger than the pool
        pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    assert e.value.code == k.api._abi.KVM_ENOMEM
    n_sel.fill_(-4)
    with pytest.raises(k.KvmError) as e:          # invalid selection from kvm_select
        pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    assert e.value.code == k.api._abi.KVM_ERANGE


def test_empty_inputs(k, dev):
    """Empty inputs: a Mean-K build of no blocks writes nothing; scoring and
    selection of no blocks are argument errors that leave their outputs alone;
    an empty selection is an empty view that stages, launches and changes
    nothing (the resident pages stay, and the next view reuses them)."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2)
    dims, dt = k.dims_for(wl), k.KVM_BF16
    raw = gc.raw_to_device(wl, "K", 0, 8, dev)
    idx = torch.full((wl.n_layers, wl.n_kv_heads, 16, wl.head_dim), 0x1234, dtype=torch.int16,
                     device=dev)
    k.kvm_build_index(dims, dt, raw, wl.block_bytes, 3, 0, idx, 16)
    torch.cuda.synchronize()
    assert bool((idx == 0x1234).all())
    q = gc.to_dev(synth.query(wl.scaled(n_q_tokens=1)), dev)
    scores = torch.full((4,), -3.0, dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_score_blocks(dims, dt, q, 1, idx, 16, 0, 0, 0, scores, ws, ws.numel())
    assert e.value.code == k.api._abi.KVM_EINVAL
    sel = torch.full((8,), -7, dtype=torch.int32, device=dev)
    n_sel = torch.full((1,), -7, dtype=torch.int32, device=dev)
    with pytest.raises(k.KvmError) as e:
        k.kvm_select(scores, 0, 0, 0, 8, 32, sel, n_sel, sel, ws, ws.numel())
    assert e.value.code == k.api._abi.KVM_EINVAL
    torch.cuda.synchronize()
    assert bool((scores == -3.0).all()) and int(n_sel.item()) == -7
    # an empty view between two views of the same blocks
    wv = wl.scaled(budget_blocks=8, n_recent=2)
    pool, keep = _remat_setup(k, dev, wv, 32, 12, "device")
    view = torch.arange(4, 12, dtype=torch.int32, device=dev)
    n8 = torch.tensor([8], dtype=torch.int32, device=dev)
    st = pool.ctx.kvm_rematerialize(view, n8, pool.page)
    torch.cuda.synchronize()
    pg = pool.page.cpu().numpy()[:8].copy()
    before_k, before_v = pool.k_view.clone(), pool.v_view.clone()
    pool.page.fill_(-9)
    st0 = pool.ctx.kvm_rematerialize(view, torch.zeros(1, dtype=torch.int32, device=dev),
                                     pool.page)
    torch.cuda.synchronize()
    assert st0["n_sel"] == 0 and st0["hits"] == st0["misses"] == st0["rotated"] == 0
    assert st0["batches"] == 0 and st0["h2d_bytes"] == 0 and st0["d2d_bytes"] == 0
    assert bool((pool.page == -9).all())
    assert torch.equal(pool.k_view, before_k) and torch.equal(pool.v_view, before_v)
    st2 = pool.ctx.kvm_rematerialize(view, n8, pool.page)
    torch.cuda.synchronize()
    assert st["misses"] == 8 and st2["hits"] == 8 and st2["misses"] == 0 and st2["rotated"] == 0
    assert np.array_equal(pool.page.cpu().numpy()[:8], pg)
    gc.check_view(wv, np.arange(4, 12), pg, pool)
    pool.ctx.close()


@pytest.mark.parametrize("T", [77, 1])
def test_scoring_and_selection_replay_in_a_hip_graph(k, dev, T):
    """Scoring (T = 77: the two matrix-core passes; T = 1: the stored-score
    form) and the allocation-free selector enqueue only kernels on the
    caller's stream, so they can be captured in a HIP graph. Five replays,
    each after new queries are copied into the captured buffer and with eager
    scoring and selection on other buffers in between, equal the eager results
    for the same queries bit for bit."""
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, n_q_tokens=T)
    N, budget = 1000, 64
    say("hip graph replay", T)
    raw = gc.raw_to_device(wl, "K", 0, N, dev)
    idx = gc.build_index_dev(k, wl, raw, dev)
    dims, dt = k.dims_for(wl), k.KVM_BF16
    ws_b = k.kvm_score_ws_bytes(dims, dt, T, N, 0, 0)
    ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
    qs = [gc.to_dev(synth.query(wl.scaled(seed=wl.seed + 100 + t)), dev) for t in range(5)]
    q = qs[0].clone()

    def bufs():
        return (torch.empty(N, dtype=torch.float32, device=dev),
                torch.empty(budget, dtype=torch.int32, device=dev),
                torch.empty(1, dtype=torch.int32, device=dev),
                torch.empty(budget, dtype=torch.int32, device=dev))

    def run(qq, out):
        sc, se, ns, bs = out
        k.kvm_score_blocks(dims, dt, qq, T, idx, N, N, 0, 0, sc, ws, ws_b)
        k.kvm_select_noalloc(sc, N, 1, 8, budget, wl.block_tokens, se, ns, bs)

    cap = bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(q, cap)                               # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(q, cap)
    eager = bufs()
    for t in range(5):
        q.copy_(qs[t])
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in cap]
        run(qs[t], eager)
        torch.cuda.synchronize()
        for a, b in zip(got, eager):
            assert torch.equal(a, b), t
        n = int(got[2].item())
        assert n == budget
        want = select_blocks(got[0].cpu().numpy().astype(np.float64), 1, 8, budget)
        assert np.array_equal(got[1].cpu().numpy()[:n], want)
    del g


# ------------------------------------------------------------ end to end ----

@pytest.mark.parametrize("name", ["tiny", "ctx64k", "ctx64k_fp8"])
def test_end_to_end_step(k, dev, name):
    import torch
    wl = synth.get_workload(name)
    N = wl.n_blocks
    say("end to end", name)
    ref = op.run_step(wl)
    raw_k = gc.raw_to_device(wl, "K", 0, N, dev)
    raw_v = gc.raw_to_device(wl, "V", 0, N, dev)
    idx = gc.build_index_dev(k, wl, raw_k, dev)
    assert np.array_equal(gc.as_f64(gc.to_host_bits(idx)), ref["index"])
    q = gc.to_dev(op.query_stored(wl, 0, ref["index"]), dev)
    scores = gc.score_dev(k, wl, q, idx, N, N, dev)
    R = scores.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(R - ref["R"]) / ref["R"]) <= 1e-5
    sel, n_sel, base = gc.select_dev(k, scores, N, wl.n_sink, wl.n_recent, wl.budget_blocks, dev)
    n = int(n_sel.item())
    say("margin", ref["margin"])
    if ref["margin"] > 2e-5:
        assert np.array_equal(sel.cpu().numpy()[:n], ref["sel"])
    gc.check_selection(sel.cpu().numpy()[:n], ref["R"], wl.n_sink, wl.n_recent, wl.budget_blocks)
    assert np.array_equal(base.cpu().numpy()[:n], ref["base_pos"])
    pool = gc.Pool(k, wl, wl.budget_blocks + 8, N, wl.budget_blocks * wl.block_tokens, dev)
    pool.ctx.kvm_ctx_set_source(0, N, raw_k, raw_v, wl.block_bytes, k.KVM_SRC_DEVICE)
    pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    torch.cuda.synchronize()
    s = sel.cpu().numpy()[:n]
    pg = pool.page.cpu().numpy()[:n]
    blocks = range(n) if n <= 64 else sorted(set(np.linspace(0, n - 1, 48).astype(int)))
    gc.check_view(wl, s, pg, pool, blocks=blocks)
    pool.ctx.close()


def test_device_backed_page_released_when_source_changes(k, dev):
    import torch
    wl = synth.get_workload("tiny")
    pool, keep = _remat_setup(k, dev, wl, 128, 16)        # device-resident sources
    sel = torch.tensor(list(range(11)), dtype=torch.int32, device=dev)
    n_sel = torch.tensor([11], dtype=torch.int32, device=dev)
    pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    torch.cuda.synchronize()
    assert pool.ctx.kvm_ctx_block_state(3)[0] >= 0
    # block 3's page is re-encoded from its device copy; moving the copy reclaims it
    rk, rv = keep
    k3, v3 = rk[3].clone(), rv[3].clone()            # same block, new location
    pool.ctx.kvm_ctx_set_source(3, 1, k3, v3, wl.block_bytes, k.KVM_SRC_DEVICE)
    assert pool.ctx.kvm_ctx_block_state(3)[0] == -1
    # a registered (shadow-backed) block keeps its page when its source changes
    pool.ctx.kvm_ctx_register_resident(50, 1, rk[50], rv[50], wl.block_bytes)
    pool.ctx.kvm_ctx_set_source(50, 1, rk[50], rv[50], wl.block_bytes, k.KVM_SRC_DEVICE)
    assert pool.ctx.kvm_ctx_block_state(50)[0] >= 0
    st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    torch.cuda.synchronize()
    assert st["misses"] == 1 and st["hits"] == 10
    gc.check_view(wl, sel.cpu().numpy(), pool.page.cpu().numpy()[:11], pool)
    pool.ctx.close()


# ----------------------------------- bounded pool: registration, rollback ----

def _state(pool, blocks):
    return {int(b): tuple(pool.ctx.kvm_ctx_block_state(int(b))) for b in blocks}


def test_register_never_takes_pages_of_the_current_view(k, dev):
    """A tight pool (the view plus three pages): freshly prefilled blocks take
    free pages or pages of blocks outside the current view and never a page
    of the view (KVMem Sec. 4.4); with only view pages left the registration
    fails with KVM_ENOMEM and changes nothing. Hits, misses and evictions
    follow the oracle's page-pool model; every view page holds its block."""
    import torch
    from oracle import PagePool
    wl = synth.get_workload("tiny")
    N, n_slots = 128, 14
    pool, keep = _remat_setup(k, dev, wl, N, n_slots)
    rk, rv = keep
    model = PagePool(n_slots)

    def update(blocks):
        sel = torch.tensor(blocks, dtype=torch.int32, device=dev)
        n_sel = torch.tensor([len(blocks)], dtype=torch.int32, device=dev)
        st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
        torch.cuda.synchronize()
        r = model.update(blocks)
        assert (st["hits"], st["misses"], st["evicted"]) == (
            len(r["hits"]), len(r["misses"]), len(r["evicted"]))
        gc.check_view(wl, np.array(blocks), pool.page.cpu().numpy()[:len(blocks)], pool)
        return sel, n_sel

    def register(b):
        pool.ctx.kvm_ctx_register_resident(b, 1, rk[b], rv[b], wl.block_bytes)
        torch.cuda.synchronize()
        model.register([b])

    view1 = list(range(0, 11))
    update(view1)
    for b in (100, 101, 102):                       # the three free pages
        register(b)
    before = _state(pool, range(N))
    with pytest.raises(k.KvmError) as e:             # only pages of the current view remain
        pool.ctx.kvm_ctx_register_resident(103, 1, rk[103], rv[103], wl.block_bytes)
    assert e.value.code == k.api._abi.KVM_ENOMEM
    assert _state(pool, range(N)) == before
    gc.check_view(wl, np.array(view1), pool.page.cpu().numpy()[:11], pool)
    view2 = [0, 1, 3, 5, 7, 9, 100, 110, 111, 126, 127]
    update(view2)                                   # 2, 4, ... 101, 102 leave the view
    for b in (103, 104):                            # LRU pages outside the view
        register(b)
    resident = {b for b in range(N) if pool.ctx.kvm_ctx_block_state(b)[0] >= 0}
    assert resident == model.resident
    gc.check_view(wl, np.array(view2), pool.page.cpu().numpy()[:11], pool)
    update([0, 1, 3, 103, 104, 110, 111, 120, 121, 126, 127])
    pool.ctx.close()


def test_register_list_matches_per_block_registration(k, dev):
    """kvm_ctx_register_resident_list: non-consecutive blocks whose raw K/V are
    packed in one buffer take the same pages as one-block registrations (the
    page rule of the oracle's pool model), their shadow and V pages hold the
    raw bytes, and the next view built from them matches the oracle. Also the
    copy launches in groups of 448 blocks (a 500-block list), the per-page copy
    path for sources that are not 16-byte aligned, a list that does not fit
    (KVM_ENOMEM, nothing changed) and malformed lists (KVM_EINVAL)."""
    import torch
    from oracle import PagePool
    wl = synth.get_workload("tiny")                 # 16 KiB pages
    N, n_slots = 1000, 600
    a, keep = _remat_setup(k, dev, wl, N, n_slots)
    b, _ = _remat_setup(k, dev, wl, N, n_slots)
    rk, rv = keep
    model = PagePool(n_slots)
    view = list(range(0, 11))
    sel = torch.tensor(view, dtype=torch.int32, device=dev)
    n_sel = torch.tensor([len(view)], dtype=torch.int32, device=dev)
    for p in (a, b):
        p.ctx.kvm_rematerialize(sel, n_sel, p.page)
    model.update(view)
    torch.cuda.synchronize()

    def packed(ids):
        return rk[ids].contiguous(), rv[ids].contiguous()

    def same_bytes(x, y):
        return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))

    ids = [3, 20, 33, 57, 90, 91, 120, 999]          # 3 is in the view: refreshed in place
    pk, pv = packed(ids)
    a.ctx.kvm_ctx_register_resident_list(ids, pk, pv, wl.block_bytes)
    for i in ids:
        b.ctx.kvm_ctx_register_resident(i, 1, rk[i], rv[i], wl.block_bytes)
    model.register(ids)
    torch.cuda.synchronize()
    assert _state(a, range(N)) == _state(b, range(N))
    resident = {i for i in range(N) if a.ctx.kvm_ctx_block_state(i)[0] >= 0}
    assert resident == model.resident
    for i in ids:
        slot = a.ctx.kvm_ctx_block_state(i)[0]
        assert same_bytes(a.k_shadow[slot], rk[i]) and same_bytes(a.v_view[slot], rv[i])
    # 500 more blocks in one list: two copy launches (448 + 52)
    big = list(range(300, 800))
    bk, bv = packed(big)
    a.ctx.kvm_ctx_register_resident_list(big, bk, bv, wl.block_bytes)
    model.register(big)
    torch.cuda.synchronize()
    for i in big[::7] + [big[447], big[448], big[-1]]:
        slot = a.ctx.kvm_ctx_block_state(i)[0]
        assert slot >= 0
        assert same_bytes(a.k_shadow[slot], rk[i]) and same_bytes(a.v_view[slot], rv[i])
    # sources 4 bytes off 16-byte alignment, stride a page plus 4 bytes: per-page copies
    odd = [40, 41, 700]
    stride = wl.block_bytes + 4
    raw = torch.zeros(len(odd) * stride + 16, dtype=torch.uint8, device=dev)
    rawv = torch.zeros_like(raw)
    for j, i in enumerate(odd):
        raw[4 + j * stride:4 + j * stride + wl.block_bytes] = rk[i].view(torch.uint8)
        rawv[4 + j * stride:4 + j * stride + wl.block_bytes] = rv[i].view(torch.uint8)
    a.ctx.kvm_ctx_register_resident_list(odd, raw[4:], rawv[4:], stride)
    model.register(odd)
    torch.cuda.synchronize()
    for i in odd:
        slot = a.ctx.kvm_ctx_block_state(i)[0]
        assert same_bytes(a.k_shadow[slot], rk[i]) and same_bytes(a.v_view[slot], rv[i])
    resident = {i for i in range(N) if a.ctx.kvm_ctx_block_state(i)[0] >= 0}
    assert resident == model.resident
    # the next view is built from the registered raw K
    view2 = [0, 3, 20, 33, 41, 57, 90, 120, 300, 747, 999]
    sel2 = torch.tensor(view2, dtype=torch.int32, device=dev)
    st = a.ctx.kvm_rematerialize(sel2, n_sel, a.page)
    torch.cuda.synchronize()
    r = model.update(view2)
    assert (st["hits"], st["misses"], st["evicted"]) == (
        len(r["hits"]), len(r["misses"]), len(r["evicted"]))
    gc.check_view(wl, np.array(view2), a.page.cpu().numpy()[:11], a)
    # a list that does not fit changes nothing: the second pool holds 18
    # blocks, all in its current view (the last selection and the blocks
    # registered since), so 582 free pages are all that can be had
    before = _state(b, range(N))
    many = [i for i in range(N) if before[i][0] < 0][:583]
    mk, mv = packed(many)
    with pytest.raises(k.KvmError) as e:
        b.ctx.kvm_ctx_register_resident_list(many, mk, mv, wl.block_bytes)
    assert e.value.code == k.api._abi.KVM_ENOMEM
    assert _state(b, range(N)) == before
    b.ctx.kvm_ctx_register_resident_list(many[:582], mk[:582], mv[:582], wl.block_bytes)
    torch.cuda.synchronize()
    assert all(b.ctx.kvm_ctx_block_state(i)[0] >= 0 for i in many[:582] + view + ids)
    before = _state(a, range(N))
    for bad in ([5, 5], [7, 6], [-1], [N]):
        bk_, bv_ = packed([0] * len(bad))
        with pytest.raises(k.KvmError) as e:
            a.ctx.kvm_ctx_register_resident_list(bad, bk_, bv_, wl.block_bytes)
        assert e.value.code == k.api._abi.KVM_EINVAL
    assert _state(a, range(N)) == before
    a.ctx.close()
    b.ctx.close()


def test_failed_gather_rolls_back_and_a_retry_is_exact(k, dev):
    """The gather callback fails on the second staging batch: the call returns
    an error after the first batch was queued. Blocks whose pages were
    completed stay resident; the others are released. Retrying the same
    selection stages only the released blocks, and every page of the view
    matches the oracle (K re-RoPE'd, V bit-exact)."""
    import ctypes
    import torch
    wl = synth.get_workload("ctx64k").scaled(n_layers=2, budget_blocks=96, n_recent=8)
    N = 400
    pool = gc.Pool(k, wl, 130, N, wl.budget_blocks * wl.block_tokens, dev, 16, 32)
    R = synth.scores_f32(21, N)
    sel, n_sel, base = gc.select_dev(k, gc.to_dev(R, dev), N, wl.n_sink, wl.n_recent,
                                     wl.budget_blocks, dev)
    s = sel.cpu().numpy()[:96]
    bad = {int(b) for b in s[16:32]}                 # the second batch of 16
    fail = [True]

    def gather(block, which, dst):
        if fail[0] and block in bad:
            return 1
        buf = (ctypes.c_char * wl.block_bytes).from_address(dst)
        arr = np.frombuffer(buf, dtype=gc.np_elem(wl))
        synth.kv_blocks(wl, "K" if which == 0 else "V", block, 1, out=arr, nthreads=1)
        return 0
    pool.ctx.kvm_ctx_set_gather(0, N, gather)
    with pytest.raises(k.KvmError) as e:
        pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    assert e.value.code == k.api._abi.KVM_ERANGE
    torch.cuda.synchronize()
    resident = [pool.ctx.kvm_ctx_block_state(int(b))[0] >= 0 for b in s]
    assert all(resident[:16]) and not any(resident[16:])
    fail[0] = False
    st = pool.ctx.kvm_rematerialize(sel, n_sel, pool.page)
    torch.cuda.synchronize()
    assert st["hits"] == 16 and st["misses"] == 80
    gc.check_view(wl, s, pool.page.cpu().numpy()[:96], pool)
    pool.ctx.close()


# ------------------------------------------------------- measured rates ----

def test_measure_rate_kinds(k, dev):
    """kvm_measure_rate: the copy moves the bytes it claims (scratch + n holds
    scratch's first n bytes), every rate is finite and within the physically
    possible range for one MI355X (below its datasheet peaks, above a tenth of
    them), and malformed requests return KVM_EINVAL."""
    import torch
    n = 64 << 20
    scratch = torch.zeros(2 * n, dtype=torch.uint8, device=dev)
    scratch[:n] = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev)
    r = k.kvm_measure_rate(k.KVM_RATE_COPY, n, scratch)
    torch.cuda.synchronize()
    assert torch.equal(scratch[n:], scratch[:n])
    assert 0.8e12 < r < 8.0e12
    sink = torch.empty(4 << 20, dtype=torch.uint8, device=dev)
    assert 0.25e15 < k.kvm_measure_rate(k.KVM_RATE_MFMA_BF16, 2000, sink) < 2.5e15
    # v_exp_f32 on 64 lanes at 2.4 GHz on 1024 SIMDs: at most 1024 * 2.4e9 * 64 / 4
    assert 1e12 < k.kvm_measure_rate(k.KVM_RATE_EXP, 2000, sink) < 1024 * 2.4e9 * 16
    # the mix's MFMA work alone bounds its score rate: 128 elements per 32 cycles
    mix = k.kvm_measure_rate(k.KVM_RATE_SCORE_MIX, 4000, sink)
    assert 0.5e12 < mix < 1024 * 2.4e9 * 128 / 32
    for kind, nn, buf in ((7, 16, sink), (k.KVM_RATE_COPY, 17, scratch),
                          (k.KVM_RATE_COPY, 2 * n, scratch), (k.KVM_RATE_EXP, 0, sink),
                          (k.KVM_RATE_EXP, 10, sink[:1024])):
        with pytest.raises(k.KvmError) as e:
            k.kvm_measure_rate(kind, nn, buf)
        assert e.value.code == k.api._abi.KVM_EINVAL
