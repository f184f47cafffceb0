"""Pins of the oracle's byte accounting against figures printed on the pages."""
import os

from oracle import kv_bytes, index_bytes

HERE = os.path.dirname(os.path.abspath(__file__))


def load():
    vals = {}
    with open(os.path.join(HERE, "golden", "page_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value = [x.strip() for x in line.split("|")[:2]]
                vals[name] = float(value)
    return vals


def test_inferscale_storage_cost_llama8b():
    v = load()
    got = kv_bytes(32, 1024, 8, 128, 2)
    assert got == 128 * 2**20                      # exactly 128 MiB
    assert abs(got / 2**20 - v["inferscale_kv_1024_tokens_llama8b"]) < 1e-9


def test_kvmem_index_grows_linearly_in_blocks():
    v = load()
    B = int(v["kvmem_block_tokens"])
    # any model with 32 KiB of index per block reproduces both Table 4 rows
    per_block = index_bytes(1, 16, 4, 256, 2)
    small = index_bytes(256 * 1024 // B, 16, 4, 256, 2) / 2**30
    large = index_bytes(10_000_000 // B, 16, 4, 256, 2) / 2**30
    assert per_block == 32 * 1024
    assert abs(small - v["kvmem_index_256k_tokens"]) <= 0.005
    assert abs(large - v["kvmem_index_10m_tokens"]) <= 0.05
