"""Input generator: determinism, layouts, poison placement, algorithmic counts."""
import numpy as np
import torch

from workloads import WORKLOADS, algorithmic_counts, draw_seqlens, make_inputs


def test_tiny_is_deterministic_and_shaped():
    a = make_inputs("tiny", 0)
    b = make_inputs("tiny", 0)
    assert torch.equal(a.q, b.q) and torch.equal(a.kvcache, b.kvcache)
    assert torch.equal(a.block_table, b.block_table)
    assert a.q.shape == (2, 1, 16, 576) and a.q.dtype == torch.bfloat16
    assert a.kvcache.shape == (8, 64, 1, 576)
    assert a.block_table.shape == (2, 3) and a.block_table.dtype == torch.int32
    assert a.cache_seqlens.tolist() == [37, 130]
    bt = a.block_table.numpy()
    assert bt[0, 1] == -1 and bt[0, 2] == -1
    used = [bt[0, 0], *bt[1]]
    assert len(set(used)) == 4 and all(0 <= p < 8 for p in used)
    c = make_inputs("tiny", 1)
    assert not torch.equal(a.q, c.q)


def test_poison_only_touches_unreadable_slots():
    x = make_inputs("tiny", 0, poison=True)
    kv = x.kvcache.float()
    bt = x.block_table.numpy()
    L = x.cache_seqlens.numpy()
    for b in range(2):
        for j in range(L[b]):
            assert torch.isfinite(kv[bt[b, j // 64], j % 64]).all()
    assert torch.isnan(kv[bt[0, 0], 37:]).all()
    assert torch.isnan(kv[bt[1, 2], 130 - 128:]).all()
    unused = set(range(8)) - {bt[0, 0], *bt[1]}
    for p in unused:
        assert torch.isnan(kv[p]).all()


def test_seqlen_rules():
    rng = np.random.Generator(np.random.PCG64(0))
    L = draw_seqlens(WORKLOADS["var_len"], rng)
    assert L.shape == (128,) and L.min() >= 1 and L.max() <= 16384
    rng = np.random.Generator(np.random.PCG64(0))
    L = draw_seqlens(WORKLOADS["skewed"], rng)
    assert (L == 131072).sum() == 1
    short = L[L != 131072]
    assert short.min() >= 512 and short.max() <= 2048


def test_algorithmic_counts_mem_bound():
    w = WORKLOADS["mem_bound"]
    c = algorithmic_counts(w, np.full(64, 4096), 64)
    assert c["kv_bytes"] == 301_989_888
    assert c["total_bytes"] == 319_865_088
    assert c["flops"] == 2 * 64 * 4096 * 128 * (576 + 512)


def test_algorithmic_counts_causal():
    w = WORKLOADS["causal_sq2"]
    c = algorithmic_counts(w, np.full(132, 8192), 128)
    assert c["visible_pairs_per_head"] == 132 * (8191 + 8192)
