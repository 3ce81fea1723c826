"""The cache append on the GPU against the oracle's kvcache_append_ref.

A copy, so the bar is bit-exact: the whole cache after the call, and the
count of rows that had no valid page.  Then a decode over the appended
cache against the oracle's decode over the oracle's appended cache."""
import numpy as np
import pytest
import torch

from oracle.mla_oracle import kvcache_append_ref
from paged_mla_decode_03_amd import MlaError, kvcache_append
from tests.gpu_helpers import DEV, MAX_ABS_LSE, MAX_ABS_O, MEAN_ABS_O, oracle, run_gpu
from workloads import WORKLOADS, DecodeInputs, Workload, make_append_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _append_and_check(inp, kv_new, bt=None):
    """Append on the GPU and compare the whole cache and the bad-row count."""
    bt = inp.block_table if bt is None else bt
    print(f"[append] B={kv_new.shape[0]} s_new={kv_new.shape[1]} h_kv={kv_new.shape[2]} "
          f"pages={inp.kvcache.shape[0]}", flush=True)
    kv = inp.kvcache.to(DEV)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvcache_append(kv_new.to(DEV), kv, bt.to(DEV), inp.cache_seqlens.to(DEV), bad)
    torch.cuda.synchronize()
    want, want_bad = kvcache_append_ref(_bits(inp.kvcache), bt.numpy(), inp.cache_seqlens.numpy(), _bits(kv_new))
    assert int(bad.item()) == want_bad
    assert np.array_equal(_bits(kv), want)
    return kv


@pytest.mark.parametrize("seqlens,s_new,h_kv", [
    ([0, 1, 63, 64, 65, 127, 128, 200], 1, 1),
    ([0, 63, 64, 4000], 2, 1),                  # two new tokens, one crossing a page boundary
    ([5, 62, 130], 3, 2),                       # two latent heads
    ([0, 10, 63], 70, 1),                       # more new tokens than a page
])
def test_append_parity(seqlens, s_new, h_kv):
    w = Workload(name="append", batch=len(seqlens), s_q=1, h_q=16 * h_kv, h_kv=h_kv,
                                       causal=False)
    inp, kv_new = make_append_inputs(w, 11, s_new, seqlens=seqlens, extra_pages=3)
    _append_and_check(inp, kv_new)


@pytest.mark.parametrize("name,s_new", [("mem_bound", 1), ("causal_sq2", 2)])
def test_append_full_size(name, s_new):
    """The decode workloads' shapes: one (or two) new tokens per sequence."""
    w = WORKLOADS[name]
    L = np.full(w.batch, (w.seqlens[0] if w.seqlens else 4096) - s_new, dtype=np.int64)
    inp, kv_new = make_append_inputs(w, 5, s_new, seqlens=L)
    _append_and_check(inp, kv_new)


def test_append_rows_without_pages():
    """Negative lengths, positions past the block table and page ids outside
    the pool are skipped (never written) and counted."""
    w = Workload(name="append", batch=4, s_q=1, h_q=16, h_kv=1, causal=False)
    inp, kv_new = make_append_inputs(w, 13, 2, seqlens=[63, 10, 20, 127], extra_pages=2)
    bt = inp.block_table.clone()
    P = inp.kvcache.shape[0]
    bt[0, 1] = -1                 # sequence 0: its second new token has no page
    bt[1, 0] = P                  # sequence 1: page id one past the pool
    inp.cache_seqlens[2] = -5     # sequence 2: negative length
    assert bt.shape[1] == 3
    inp.cache_seqlens[3] = 191    # sequence 3: position 191 has a page, 192 lies past the table
    _append_and_check(inp, kv_new, bt)


def test_append_rejects_bad_tensors():
    w = Workload(name="append", batch=2, s_q=1, h_q=16, h_kv=1, causal=False)
    inp, kv_new = make_append_inputs(w, 1, 1, seqlens=[3, 4])
    kv = inp.kvcache.to(DEV)
    with pytest.raises(TypeError):
        kvcache_append(kv_new.float().to(DEV), kv, inp.block_table.to(DEV), inp.cache_seqlens.to(DEV))
    with pytest.raises(ValueError):
        kvcache_append(kv_new[:, :, :, :512].contiguous().to(DEV), kv, inp.block_table.to(DEV),
                       inp.cache_seqlens.to(DEV))


@pytest.mark.parametrize("name", ["mem_bound", "causal_sq2"])
def test_append_then_decode(name):
    """Append the step's new tokens, advance the lengths, decode: the result
    matches the oracle's decode over the oracle's appended cache (sampled
    sequences at the full size)."""
    w = WORKLOADS[name]
    s_new = w.s_q
    L = np.full(w.batch, (w.seqlens[0] if w.seqlens else 4096) - s_new, dtype=np.int64)
    inp, kv_new = make_append_inputs(w, 17, s_new, seqlens=L)
    print(f"[append+decode] {name}", flush=True)
    kv = _append_and_check(inp, kv_new)
    L_after = inp.cache_seqlens + s_new
    want_kv, _ = kvcache_append_ref(_bits(inp.kvcache), inp.block_table.numpy(), inp.cache_seqlens.numpy(),
                                    _bits(kv_new))
    after = DecodeInputs(inp.workload, 17, inp.q, torch.from_numpy(want_kv.view(np.int16)).view(torch.bfloat16),
                         inp.block_table, L_after)
    o, lse, _, _ = run_gpu(after, dev_tensors=(inp.q.to(DEV), kv, inp.block_table.to(DEV), L_after.to(DEV)))
    subset = [0, w.batch // 2, w.batch - 1]
    O, LSE = oracle(after, batch_subset=subset)
    for b in subset:
        d = np.abs(o[b] - O[b])
        assert d.max() <= MAX_ABS_O and d.mean() <= MEAN_ABS_O
        assert np.abs(lse[b] - LSE[b]).max() <= MAX_ABS_LSE
