"""The whole-page allocator on the GPU (mla_pages_* through the C ABI):
bit-exact against the oracle over random sequences of reserves and
releases (free stack, counter, block table and status after every call),
and end to end: pages reserved, new tokens appended into them, and the
decode over the resulting tables checked against the decode oracle."""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from gpu_helpers import DEV, compare
from paged_mla_decode_03_amd import PagePool, get_mla_metadata, kvcache_append, mla_decode_paged
from workloads import bf16_normal

pytestmark = pytest.mark.gpu


def _walk(seed, B, P, max_pages, steps, max_new):
    rng = np.random.default_rng(seed)
    pool = PagePool(P, DEV)
    fp, cnt = mo.pages_init_ref(P)
    bt_ref = np.full((B, max_pages), -1, dtype=np.int64)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32, device=DEV)
    L = np.zeros(B, dtype=np.int64)
    statuses = set()
    for step in range(steps):
        Ld = torch.from_numpy(L.astype(np.int32)).to(DEV)
        if rng.random() < 0.7:
            s_new = int(rng.integers(0, max_new))
            fp, cnt, bt_ref, st, n = mo.pages_reserve_ref(fp, cnt, L, s_new, bt_ref)
            pool.reserve(Ld, s_new, bt)
            if st == 0:
                L = L + s_new
        else:
            rel = (rng.random(B) < 0.3).astype(np.int32)
            fp, cnt, bt_ref, st, n = mo.pages_release_ref(fp, cnt, L, rel, bt_ref, P)
            pool.release(Ld, torch.from_numpy(rel).to(DEV), bt)
            if st == 0:
                L = np.where(rel != 0, 0, L)
        statuses.add(st)
        g_cnt, g_st, g_n = pool.status()
        assert (g_cnt, g_st) == (cnt, st), f"step {step}: GPU ({g_cnt}, {g_st}) vs oracle ({cnt}, {st})"
        if st != 2:
            assert g_n == n, f"step {step}: pages moved {g_n} vs {n}"
        assert np.array_equal(bt.cpu().numpy(), bt_ref), f"step {step}: block tables differ"
        assert np.array_equal(pool.free_pages[:cnt].cpu().numpy(), fp[:cnt]), f"step {step}: free stacks differ"
    return statuses


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_allocator_bit_exact_small(seed):
    statuses = _walk(seed, B=5, P=40, max_pages=12, steps=80, max_new=150)
    assert 0 in statuses and 1 in statuses


def test_allocator_bit_exact_large_batch():
    """More sequences than the kernel's 1024 threads: the scans carry over
    chunks."""
    _walk(7, B=1500, P=30000, max_pages=40, steps=12, max_new=300)


def test_allocator_refuses_out_of_range_and_double_release():
    P, B, mp = 16, 3, 4
    pool = PagePool(P, DEV)
    bt = torch.full((B, mp), -1, dtype=torch.int32, device=DEV)
    L = torch.tensor([0, 10, 0], dtype=torch.int32, device=DEV)
    pool.reserve(L, 300, bt)                       # 5 pages > max_pages 4
    assert pool.status() == (P, 2, 0) and (bt == -1).all()
    pool.reserve(L, 200, bt)                       # 4, 3 (one page counted as mapped), 4: 11 of 16
    assert pool.status() == (5, 0, 11)
    L2 = L + 200
    rel = torch.tensor([1, 0, 0], dtype=torch.int32, device=DEV)
    pool.release(L2, rel, bt)
    assert pool.status() == (9, 0, 4)
    pool.release(L2, rel, bt)                      # again: its entries are -1 now
    assert pool.status() == (9, 2, 0)


@pytest.mark.parametrize("s_q,h_q", [(1, 128), (2, 64)])
def test_reserve_append_decode_end_to_end(s_q, h_q):
    """Three sequences prefilled with 100 tokens, then decode steps of s_q
    new tokens each: reserve, append, decode.  Midway sequence 1 finishes,
    its pages go back, and a new sequence starts in its slot and reuses
    them.  Every few steps the decode is checked against the oracle run on
    the tables and cache the GPU holds."""
    rng = np.random.Generator(np.random.PCG64(5))
    B, P, mp = 3, 24, 6
    pool = PagePool(P, DEV)
    kv = torch.zeros((P, 64, 1, 576), dtype=torch.bfloat16, device=DEV)
    bt = torch.full((B, mp), -1, dtype=torch.int32, device=DEV)
    L = np.zeros(B, dtype=np.int64)

    def step(s_new):
        nonlocal L
        Ld = torch.from_numpy(L.astype(np.int32)).to(DEV)
        pool.reserve(Ld, s_new, bt)
        assert pool.status()[1] == 0
        kv_new = bf16_normal(rng, (B, s_new, 1, 576)).to(DEV)
        kvcache_append(kv_new, kv, bt, Ld)
        L = L + s_new

    step(100)
    checked = 0
    for t in range(70):
        step(s_q)
        if t == 30:   # sequence 1 ends; a new one starts in its slot
            Ld = torch.from_numpy(L.astype(np.int32)).to(DEV)
            pool.release(Ld, torch.tensor([0, 1, 0], dtype=torch.int32, device=DEV), bt)
            assert pool.status()[1] == 0
            L[1] = 0
            step(s_q)
        if t % 10 == 9:
            Ld = torch.from_numpy(L.astype(np.int32)).to(DEV)
            q = bf16_normal(rng, (B, s_q, h_q, 576))
            meta, ns = get_mla_metadata(Ld, s_q * h_q, 1)
            o, lse = mla_decode_paged(q.to(DEV), kv, bt, Ld, 512, meta, ns, causal=True)
            torch.cuda.synchronize()
            O, LSE = mo.mla_decode_ref(q, kv.cpu(), bt.cpu().numpy(), L, 512, causal=True)
            compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), O, LSE,
                    label=f"step {t} L={L.tolist()}")
            checked += 1
    # every page is either free or mapped by exactly one live block
    cnt = pool.status()[0]
    mapped = [int(x) for b in range(B) for x in bt[b, :(int(L[b]) + 63) // 64].tolist()]
    assert sorted(mapped + pool.free_pages[:cnt].tolist()) == list(range(P))
    assert checked == 7
