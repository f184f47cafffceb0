"""The library's host-only C++ (block pool, rematerialization data plane, host
tier) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
driven through tests/host/pool_driver.cpp with a fake device (KVMem Sec. 4.4:
bounded page pool, delta working sets, pipelined staging; Fig. 3).

Checked against the oracle: hits, misses and evictions of every working-set
update against oracle.plan.PagePool, the resident set G_t, and the host-tier
counts against oracle.simulate_host_tier. Checked by the driver itself: every
view page holds its block at its compact position, no kernel runs before the
copies into its source, and no staging half is refilled while a copy from it
is queued (the fake device runs copies as late as the events allow and the
gather workers finish in a shuffled order). Failures injected into launches,
copies and gather callbacks must leave every resident page consistent with
its record, and the retry must give an exact view. A corrupted source byte of
V must be reported. A pool too large for host memory gives KVM_ENOMEM.
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import PagePool, simulate_host_tier

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_space_block_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("host_common.cpp", "pool.cpp", "dataplane.cpp",
                                            "tier.cpp")]
DRIVER = os.path.join(ROOT, "tests", "host", "pool_driver.cpp")
KVM_ENOMEM = -2


def _build(out, sanitize):
    flags = ["-std=c++17", "-g", "-O1", "-Wall", "-Wextra", "-Wno-unused-parameter"]
    if sanitize:
        flags += ["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                  "-fno-sanitize-recover=undefined"]
    else:
        flags = ["-std=c++17", "-O2"]
    cmd = ["g++", *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SOURCES, DRIVER,
           "-o", out, "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    return _build(str(tmp_path_factory.mktemp("host") / "pool_driver_asan"), True)


@pytest.fixture(scope="module")
def driver_plain(tmp_path_factory):
    return _build(str(tmp_path_factory.mktemp("host") / "pool_driver"), False)


def run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], input="\n".join(lines + ["end"]) + "\n", capture_output=True,
                       text=True, env=env, timeout=600)
    assert p.returncode == 0, p.stderr[-4000:]
    out = p.stdout.splitlines()
    errors = [x for x in out if x.startswith("error ")]
    return [x for x in out if not x.startswith("error ")], errors


class Trace:
    """Builds a driver script and the expected pool-model results alongside."""

    def __init__(self, n_slots, max_blocks, delta, batch, staging, seed):
        self.lines = [f"pool {n_slots} {max_blocks} {delta} {batch} {staging} {seed}"]
        self.model = PagePool(n_slots)
        self.expect = []            # per output line: None or a checker

    def add(self, line, check=None):
        self.lines.append(line)
        self.expect.append(check)


def sel_line(blocks):
    return f"sel {len(blocks)} " + " ".join(str(b) for b in blocks)


def parse_sel(line):
    f = line.split()
    assert f[0] == "sel"
    rc, hits, misses, evicted, rotated, h2d_pages, batches, view_err = (int(x) for x in f[1:])
    return dict(rc=rc, hits=hits, misses=misses, evicted=evicted, rotated=rotated,
                h2d_pages=h2d_pages, batches=batches, view_errors=view_err)


def random_scenario(seed, delta, sources, fail_rate):
    rng = np.random.default_rng(seed)
    n_slots = int(rng.integers(12, 40))
    budget = int(rng.integers(4, n_slots - 4))
    max_blocks = 400
    batch = int(rng.choice([1, 3, 8]))
    staging = 2 * batch + 2 * int(rng.integers(0, 3))
    lines = [f"pool {n_slots} {max_blocks} {delta} {batch} {staging} {seed}"]
    nb = 60
    # lower tiers of the first blocks; later blocks arrive by registration
    for first in range(0, max_blocks, 20):
        kind = sources[(first // 20) % len(sources)]
        if kind == "gather":
            lines.append(f"gather {first} 20")
        else:
            lines.append(f"src {first} 20 {1 if kind == 'pinned' else 2}")
    steps = []
    for t in range(40):
        if rng.random() < 0.4:
            n_new = int(rng.integers(1, 4))
            steps.append(("reg", list(range(nb, nb + n_new))))
            nb += n_new
        if rng.random() < 0.1:
            b = int(rng.integers(0, nb))
            steps.append(("evict", [b]))
        if rng.random() < 0.2:
            # blocks staged back, not consecutive (some may be resident)
            ids = sorted(rng.choice(nb, int(rng.integers(1, 5)), replace=False).tolist())
            steps.append(("regl", ids))
        k = int(rng.integers(1, budget + 1))
        blocks = sorted(rng.choice(nb, min(k, nb), replace=False).tolist())
        fail = None
        if rng.random() < fail_rate:
            fail = (str(rng.choice(["launch", "h2d", "gather"])), int(rng.integers(1, 6)))
        steps.append(("sel", blocks, fail))
    return lines, steps, n_slots


def play(exe, lines, steps, n_slots):
    """Run the steps one driver command at a time in one process (the script
    is replayed incrementally so the model can follow rollbacks)."""
    model = PagePool(n_slots)
    script = list(lines)
    outputs_needed = []
    # first pass: run everything and collect outputs; the model is updated
    # while parsing, using `state` after each selection to follow rollbacks
    for st in steps:
        if st[0] == "reg":
            script.append(f"reg {st[1][0]} {len(st[1])}")
            outputs_needed.append(("reg", st[1]))
        elif st[0] == "regl":
            script.append("regl " + " ".join(str(x) for x in [len(st[1])] + st[1]))
            outputs_needed.append(("reg", st[1]))
        elif st[0] == "evict":
            script.append(f"evict {st[1][0]} 1")
            outputs_needed.append(("evict", st[1]))
        else:
            _, blocks, fail = st
            if fail:
                script.append(f"fail {fail[0]} {fail[1]}")
                outputs_needed.append(("fail",))
            script.append(sel_line(blocks))
            outputs_needed.append(("sel", blocks, fail))
            script.append("state")
            outputs_needed.append(("state",))
            script.append("check")
            outputs_needed.append(("check",))
    out, errors = run(exe, script)
    assert not errors, errors[:10]
    head = len(lines)
    res = out[head:]
    assert len(res) >= len(outputs_needed)
    failures = 0
    i = 0
    last_sel = None
    while i < len(outputs_needed):
        need, got = outputs_needed[i], res[i]
        if need[0] == "reg":
            rc = int(got.split()[1])
            try:
                model.register(need[1])
                assert rc == 0, got
            except Exception as e:          # PoolFull
                assert type(e).__name__ == "PoolFull" and rc == KVM_ENOMEM, got
        elif need[0] == "evict":
            assert got == "evict 0"
            model.evict(need[1])
        elif need[0] == "sel":
            r = parse_sel(got)
            blocks, fail = need[1], need[2]
            last_sel = (blocks, r)
            if r["rc"] == 0:
                m = model.update(blocks)
                assert (r["hits"], r["misses"], r["evicted"]) == (
                    len(m["hits"]), len(m["misses"]), len(m["evicted"])), (got, m)
                assert r["rotated"] <= len(blocks) and r["view_errors"] == 0
            else:
                assert fail is not None, got          # only injected failures fail
                failures += 1
        elif need[0] == "state":
            resident = {int(x) for x in got.split()[1:]}
            blocks, r = last_sel
            if r["rc"] != 0:
                # follow the rollback: the step happened, released blocks are gone
                model.step += 1
                model.last_use = {b: (model.step if b in set(blocks) else model.last_use[b])
                                  for b in resident}
            assert resident == model.resident
        elif need[0] == "check":
            assert got == "check 0", got
        i += 1
    assert res[-1] == "errors 0"
    return failures


@pytest.mark.parametrize("seed,delta,sources", [
    (1, 0, ["pinned"]), (2, 0, ["device"]), (3, 0, ["gather"]),
    (4, 0, ["pinned", "gather", "device"]), (5, 2, ["pinned", "device"]),
    (6, 1, ["gather", "pinned"]), (7, 3, ["device", "gather"]), (8, 0, ["gather", "pinned"]),
])
def test_pool_and_data_plane_follow_the_oracle_pool_model(driver, seed, delta, sources):
    lines, steps, n_slots = random_scenario(seed, delta, sources, fail_rate=0.0)
    play(driver, lines, steps, n_slots)


@pytest.mark.parametrize("seed,delta,sources", [
    (11, 0, ["gather"]), (12, 0, ["pinned"]), (13, 2, ["pinned", "gather", "device"]),
    (14, 0, ["pinned", "gather", "device"]), (15, 1, ["device", "gather"]),
])
def test_injected_failures_roll_back_to_a_consistent_pool(driver, seed, delta, sources):
    lines, steps, n_slots = random_scenario(seed, delta, sources, fail_rate=0.35)
    assert play(driver, lines, steps, n_slots) > 0


def test_gather_failure_then_retry_gives_the_exact_view(driver):
    blocks = list(range(0, 40, 2))
    script = ["pool 24 100 0 4 8 3", "gather 0 100", "fail gather 11", sel_line(blocks), "state",
              "check", sel_line(blocks), "check"]
    out, errors = run(driver, script)
    assert not errors
    first = parse_sel(out[3])
    assert first["rc"] == -4                      # the callback's failure
    resident = {int(x) for x in out[4].split()[1:]}
    # batches of 4 blocks (8 gather calls each); call 11 is in the second batch
    assert resident == set(blocks[:4])
    assert out[5] == "check 0"
    second = parse_sel(out[6])
    assert second["rc"] == 0 and second["hits"] == 4 and second["misses"] == 16
    assert second["view_errors"] == 0 and out[7] == "check 0"


def test_a_corrupted_v_source_byte_is_reported(driver):
    script = ["pool 16 50 0 4 8 9", "src 0 50 1", "corrupt 7", sel_line([1, 3, 7, 9])]
    out, errors = run(driver, script)
    r = parse_sel(out[3])
    assert r["rc"] == 0 and r["view_errors"] == 1
    assert errors == ["error view V of block 7"]


def test_pool_too_large_for_host_memory_is_enomem(driver_plain):
    out, errors = run(driver_plain, ["pool 8 16 0 4 8 1", "oom 1099511627776"])
    assert out[1] == f"oom {KVM_ENOMEM}"


def test_host_tier_matches_the_oracle_under_sanitizers(driver):
    rng = np.random.default_rng(23)
    for trial in range(6):
        steps, nb = [], 0
        script_steps = []
        for t in range(30):
            new = list(range(nb, nb + int(rng.integers(0, 4))))
            nb += len(new)
            if nb == 0:
                new, nb = [0], 1
            sel = sorted(rng.choice(nb, min(nb, int(rng.integers(1, 12))), replace=False).tolist())
            miss = sorted(b for b in sel if rng.random() < 0.4)
            steps.append((new, sel, miss))
            for lst in (new, sel, miss):
                script_steps.append(" ".join(str(x) for x in [len(lst), *lst]))
        policy = trial % 2
        cap = int(rng.integers(2, 20))
        lam = [0.0, 0.3, 1.0][trial % 3]
        out, errors = run(driver, [f"tier {policy} {cap} {lam} {len(steps)}", *script_steps])
        assert not errors
        f = [int(x) for x in out[0].split()[1:]]
        assert f[0] == 0
        got = [tuple(f[1 + 3 * i:4 + 3 * i]) for i in range(len(steps))]
        want = simulate_host_tier(steps, cap, "lru" if policy == 0 else "lrfu", lam)
        assert got == [tuple(x) for x in want]
