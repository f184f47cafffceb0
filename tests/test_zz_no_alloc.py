"""kvm_select_noalloc (no workspace argument, the library's fixed per-GPU
scratch) against kvm_select with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input, each compared bit for bit
with kvm_select and with the oracle's selector on the same fp32 scores (KVMem
Sec. 4.3 default selector: sink and recent blocks kept, top-k of the rest, ties
to the lower block id, ascending order, positions 32 i).
"""
import numpy as np
import pytest

import synth
from oracle import compact_positions, select_blocks
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _noalloc(k, scores, n, sink, recent, budget, dev):
    import torch
    sel = torch.full((budget,), -7, dtype=torch.int32, device=dev)
    n_sel = torch.zeros(1, dtype=torch.int32, device=dev)
    base = torch.full((budget,), -7, dtype=torch.int32, device=dev)
    k.kvm_select_noalloc(scores, n, sink, recent, budget, 32, sel, n_sel, base)
    return sel, n_sel, base


def _compare(k, dev, R, sink, recent, budget):
    import torch
    n = len(R)
    scores = gc.to_dev(R, dev)
    want = select_blocks(R.astype(np.float64), sink, recent, budget)
    s1, n1, b1 = gc.select_dev(k, scores, n, sink, recent, budget, dev)
    s2, n2, b2 = _noalloc(k, scores, n, sink, recent, budget, dev)
    torch.cuda.synchronize()
    m = int(n1.item())
    assert m == int(n2.item()) == min(n, budget)
    assert np.array_equal(s2.cpu().numpy()[:m], s1.cpu().numpy()[:m])
    assert np.array_equal(b2.cpu().numpy()[:m], b1.cpu().numpy()[:m])
    assert np.array_equal(s2.cpu().numpy()[:m], want)
    assert np.array_equal(b2.cpu().numpy()[:m], compact_positions(m))


def test_noalloc_select_equals_select_on_two_calls():
    import torch
    import attention_space_block_amd as k
    dev = torch.device("cuda:0")
    k._abi.lib()
    say("noalloc select: 312,500 blocks with ties (10M-token view budget)")
    _compare(k, dev, synth.scores_f32(41, 312500, kind="ties", levels=64), 1, 256, 2048)
    say("noalloc select: 5,000 blocks, second call on the same scratch")
    _compare(k, dev, synth.scores_f32(42, 5000), 1, 64, 512)
    say("noalloc select: every block selected (no scratch use)")
    _compare(k, dev, synth.scores_f32(43, 300), 1, 8, 512)


def test_noalloc_select_refuses_more_blocks_than_its_scratch():
    import torch
    import attention_space_block_amd as k
    dev = torch.device("cuda:0")
    scores = torch.zeros(16, dtype=torch.float32, device=dev)
    limit = 31326208
    with pytest.raises(k.KvmError) as e:
        _noalloc(k, scores, limit + 1, 1, 8, 100, dev)
    assert e.value.code == k.api._abi.KVM_ENOMEM
    assert "scratch" in str(e.value)
