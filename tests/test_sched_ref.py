"""CPU checks of the split-KV scheduler's reference rule.

The rule is the build's own (the pages only name the call and its outputs on
the dolphin-ai.jp FlashMLA page, "FlashMLA の使用方法", step 3, and ask for
balance over variable-length sequences in the deepseek.csdn.net article,
section 4.2(2)).  It is pinned here by an independent unit-by-unit simulation
of the cost line, and by the invariants any correct split must satisfy:
every (sequence, page) is covered exactly once, each worker stays within the
quota, split slots are dense and unique.
"""
import numpy as np
import pytest

from oracle.sched_ref import FIXED_OVERHEAD_PAGES, PAGE_SIZE, num_workers_ref, segments_of, split_rule


def simulate(seqlens, W, F):
    """Walk the cost line one unit at a time; returns per-worker segment lists
    [(b, page_lo, page_hi)] and per-sequence split counts."""
    units = []
    for b, L in enumerate(seqlens):
        units += [None] * (F // 2)
        units += [(b, p) for p in range((L + PAGE_SIZE - 1) // PAGE_SIZE)]
        units += [None] * (F - F // 2)
    T = len(units)
    Q = max(1, -(-T // W))
    segs = [[] for _ in range(W)]
    for u, item in enumerate(units):
        if item is None:
            continue
        w = u // Q
        b, p = item
        if segs[w] and segs[w][-1][0] == b and segs[w][-1][2] == p:
            segs[w][-1] = (b, segs[w][-1][1], p + 1)
        else:
            segs[w].append((b, p, p + 1))
    counts = [0] * len(seqlens)
    for w in range(W):
        for b, _, _ in segs[w]:
            counts[b] += 1
    return segs, counts, Q


CASES = [
    ([37, 130], 256),
    ([4096] * 64, 256),
    ([8192] * 132, 128),
    ([0, 1, 63, 64, 65, 0, 131072], 256),
    ([0, 0, 0], 7),
    ([1], 1),
    ([5000, 1, 1, 1, 70000], 3),
]


@pytest.mark.parametrize("seqlens,W", CASES)
@pytest.mark.parametrize("F", [0, 1, FIXED_OVERHEAD_PAGES, 5])
def test_rule_matches_unit_simulation(seqlens, W, F):
    meta, ns = split_rule(seqlens, W, F)
    segs, counts, Q = simulate(seqlens, W, F)
    assert meta.shape == (W, 8) and meta.dtype == np.int32
    assert ns.shape == (len(seqlens) + 1,) and ns.dtype == np.int32
    assert ns[0] == 0 and list(np.diff(ns)) == counts
    seen_slots = set()
    covered = {}
    for w in range(W):
        got = segments_of(meta[w], seqlens, ns)
        assert [(b, lo, hi) for b, lo, hi, _ in got] == segs[w]
        assert sum(hi - lo for _, lo, hi, _ in got) <= Q
        for b, lo, hi, slot in got:
            assert ns[b] <= slot < ns[b + 1]
            assert slot not in seen_slots
            seen_slots.add(slot)
            for p in range(lo, hi):
                assert (b, p) not in covered
                covered[(b, p)] = w
        if not got:
            assert list(meta[w]) == [0, 0, -1, 0, 0, 0, 0, 0]
    expect = {(b, p) for b, L in enumerate(seqlens) for p in range((L + PAGE_SIZE - 1) // PAGE_SIZE)}
    assert set(covered) == expect
    assert len(seen_slots) == int(ns[-1]) <= W + len(seqlens)


def test_uniform_workload_is_balanced():
    # 64 x 64 pages over 256 workers with no overhead: 16 pages each, 4 splits each.
    meta, ns = split_rule([4096] * 64, 256, 0)
    assert list(np.diff(ns)) == [4] * 64
    for w in range(256):
        (b, lo, hi, slot), = segments_of(meta[w], [4096] * 64, ns)
        assert hi - lo == 16


def test_two_workers_sharing_a_sequence_get_equal_pages():
    # 64 x 64 pages over 128 workers: every sequence is split in two, and each
    # half pays one of the sequence's two fixed costs, so all workers get 32.
    meta, ns = split_rule([4096] * 64, 128, FIXED_OVERHEAD_PAGES)
    assert list(np.diff(ns)) == [2] * 64
    for w in range(128):
        (b, lo, hi, slot), = segments_of(meta[w], [4096] * 64, ns)
        assert hi - lo == 32


def test_num_workers():
    assert num_workers_ref(256, 128, 1) == 128   # two 64-row blocks per head
    assert num_workers_ref(256, 129, 1) == 128   # two 128-row blocks
    assert num_workers_ref(256, 256, 1) == 128   # two 128-row blocks
    assert num_workers_ref(256, 384, 1) == 85    # three 128-row blocks
    assert num_workers_ref(256, 64, 1) == 256    # one 64-row block
    assert num_workers_ref(256, 65, 1) == 128    # two 64-row blocks
    assert num_workers_ref(256, 16, 1) == 256
    assert num_workers_ref(256, 64, 2) == 128
    assert num_workers_ref(80, 129, 1) == 40
    assert num_workers_ref(1, 1024, 8) == 1
