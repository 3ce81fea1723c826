"""Robustness of the HIP path: poisoned unused cache slots, page-permutation
invariance, determinism, causal reductions, and the combine kernel alone."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, compare, oracle, run_gpu, to_dev
from oracle.mla_oracle import lse_combine_ref
from paged_mla_decode_03_amd import DecodeBuffers, get_mla_metadata, mla_combine_splits, mla_decode_paged
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _custom(s_q, h_q, causal, seqlens, seed, **kw):
    w = Workload("custom", batch=len(seqlens), s_q=s_q, h_q=h_q, h_kv=1, causal=causal,
                 seqlens=tuple(seqlens), num_pages=None)
    return make_inputs(w, seed, seqlens=seqlens, **kw)


@pytest.mark.parametrize("h_q", [32, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_poisoned_unused_slots_change_nothing(causal, h_q):
    """64-row (2 x 32 rows) and 128-row (2 x 128 rows) workgroups alike."""
    lens = [37, 130, 64, 1]
    clean = _custom(2, h_q, causal, lens, 3, extra_pages=3)
    dirty = _custom(2, h_q, causal, lens, 3, extra_pages=3, poison=True)
    assert torch.isnan(dirty.kvcache.float()).any()
    a = run_gpu(clean)
    b = run_gpu(dirty)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_page_permutation_bitwise():
    inp = _custom(1, 128, False, [300, 64, 129], 4, extra_pages=5)
    a = run_gpu(inp)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(inp.kvcache.shape[0]))
    kv2 = torch.empty_like(inp.kvcache)
    kv2[perm] = inp.kvcache
    bt = inp.block_table.long()
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32)
    inp.kvcache, inp.block_table = kv2, bt2
    b = run_gpu(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_deterministic():
    inp = make_inputs("var_len", 1)
    dev = to_dev(inp)
    a = run_gpu(inp, dev_tensors=dev)
    b = run_gpu(inp, dev_tensors=dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_single_token_equals_noncausal():
    inp = _custom(1, 128, False, [77, 640, 1], 6)
    a = run_gpu(inp, causal=True)
    b = run_gpu(inp, causal=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("variant", ["wave", "wide"])
@pytest.mark.parametrize("counts", [[1, 3, 36], [2, 19, 5], [7, 13, 0], [11, 8, 22], [300, 1, 17], [2, 257, 0]])
def test_combine_kernel_alone_on_synthetic_partials(counts, variant):
    """Write partials straight into the workspace and check the merge of the
    first three sequences against the oracle's formula: a split left alone,
    an empty sequence, a split that saw no key, and many splits.  Both
    variants: one wave per row (chosen when workers <= 2 x sequences; its
    first four splits load together, then four, two, one at a time) and one
    workgroup per row (chosen when there are more workers; four waves take
    splits w, w + 4, ..., four at a time each, so 16 per round, and above 256
    splits the threads' strided reductions of the lse values wrap around).
    These counts end every round at a different place."""
    s_q, h_q, h_kv, dv = 1, 64, 1, 512
    if variant == "wide":
        full = list(counts)
        W = max(40, sum(full))
    else:
        pad = max(0, sum(counts) - 6)                # enough one-split sequences that W <= 2 B
        full = list(counts) + [1] * pad
        W = sum(full)
    B = len(full)
    assert (W > 2 * B) == (variant == "wide")
    R = s_q * h_q // h_kv
    ns = torch.tensor(np.concatenate([[0], np.cumsum(full)]), dtype=torch.int32, device=DEV)
    q = torch.zeros((B, s_q, h_q, 576), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 64, h_kv, 576), dtype=torch.bfloat16, device=DEV)
    buf = DecodeBuffers(q, kv, dv, W)
    slots = W + B
    ws = buf.workspace.view(torch.float32)
    ws_o = ws[: slots * h_kv * R * dv].view(slots, h_kv, R, dv)
    ws_l = ws[slots * h_kv * R * dv: slots * h_kv * R * (dv + 1)].view(slots, h_kv, R)
    rng = np.random.default_rng(0)
    po = rng.standard_normal((slots, h_kv, R, dv)).astype(np.float32)
    pl = rng.normal(3.0, 2.0, (slots, h_kv, R)).astype(np.float32)
    pl[int(np.cumsum(counts)[0]) + 1] = -np.inf  # a split that saw no key
    ws_o.copy_(torch.from_numpy(po))
    ws_l.copy_(torch.from_numpy(pl))
    buf.o.fill_(7.0)
    buf.lse.fill_(7.0)
    mla_combine_splits(ns, s_q, h_q, h_kv, dv, W, buf)
    torch.cuda.synchronize()
    o = buf.o.float().cpu().numpy()
    lse = buf.lse.cpu().numpy()
    for b in range(3):
        s0, n = int(ns[b]), full[b]
        if n == 1:                               # single split: left to the decode kernel
            assert (o[b] == 7.0).all() and (lse[b] == 7.0).all()
            continue
        O, L = lse_combine_ref(po[s0:s0 + n, 0].astype(np.float64), pl[s0:s0 + n, 0].astype(np.float64))
        np.testing.assert_allclose(o[b, 0], O, rtol=0, atol=2e-2 * max(1, np.abs(O).max()))
        np.testing.assert_allclose(lse[b, :, 0], L, rtol=0, atol=1e-5 * max(1, np.abs(L).max()))


def test_zero_length_sequences_write_zero_and_neg_inf():
    inp = _custom(1, 16, False, [0, 5, 0], 2)
    o, lse, _, _ = run_gpu(inp)
    assert (o[0] == 0).all() and (o[2] == 0).all()
    assert np.isneginf(lse[0]).all() and np.isneginf(lse[2]).all()
    O, LSE = oracle(inp)
    compare(o, lse, O, LSE, label="zero-length")


def test_timed_decode_matches_untimed_and_times_the_kernel():
    """mla_decode_splitkv_timed runs the same kernel (bitwise the same
    outputs) and its dispatch-recorded events bracket a positive duration."""
    from paged_mla_decode_03_amd import mla_decode_splitkv, mla_decode_splitkv_timed
    inp = _custom(1, 128, False, [70, 1300, 5], 4)
    q, kv, bt, L = to_dev(inp)
    meta, ns = get_mla_metadata(L, 128, 1, 17)
    a = DecodeBuffers(q, kv, 512, 17)
    b = DecodeBuffers(q, kv, 512, 17)
    mla_decode_splitkv(q, kv, bt, L, 512, meta, ns, buffers=a)
    mla_combine_splits(ns, 1, 128, 1, 512, 17, a)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mla_decode_splitkv_timed(q, kv, bt, L, 512, meta, ns, start, stop, buffers=b)
    mla_combine_splits(ns, 1, 128, 1, 512, 17, b)
    stop.synchronize()
    ms = start.elapsed_time(stop)
    assert 0 < ms < 1000, ms
    assert torch.equal(a.o, b.o) and torch.equal(a.lse, b.lse)
