"""The fp8 cache on the GPU: the quantizing append bit-exact against the
oracle (codes of every row, rows without a page counted), and the decode
over fp8 codes against the oracle's decode of the cache's values
decode(code) * kv_scale, with the usual bars; poisoned (NaN-code) slots
change nothing.  The decode inputs are the oracle's codes of the seeded
N(0, 1) latents at the scale 1/64."""
import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from gpu_helpers import DEV, compare, oracle_fp8_codes
from paged_mla_decode_03_amd import MlaError, get_mla_metadata, kvcache_append_fp8, mla_decode_paged_fp8
from workloads import Workload, bf16_normal, make_append_inputs, make_fp8_inputs

pytestmark = pytest.mark.gpu


def _custom(s_q, h_q, h_kv, causal, seqlens, seed, **kw):
    w = Workload("custom", batch=len(seqlens), s_q=s_q, h_q=h_q, h_kv=h_kv, causal=causal,
                 seqlens=tuple(seqlens), num_pages=None)
    return make_fp8_inputs(w, seed, encode=oracle_fp8_codes, seqlens=seqlens, **kw)


def _run(inp, num_workers=None):
    w = inp.workload
    q, kv, bt, L = (inp.q.to(DEV), inp.kvcache.to(DEV), inp.block_table.to(DEV), inp.cache_seqlens.to(DEV))
    meta, ns = get_mla_metadata(L, w.s_q * w.h_q // w.h_kv, w.h_kv, num_workers)
    o, lse = mla_decode_paged_fp8(q, kv, inp.extra["kv_scale"], bt, L, 512, meta, ns, causal=w.causal)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy(), np.diff(ns.cpu().numpy())


def _oracle(inp, batch_subset=None):
    return mo.mla_decode_fp8_ref(inp.q, inp.kvcache.numpy(), inp.extra["kv_scale"], inp.block_table.numpy(),
                                 inp.cache_seqlens.numpy(), 512, causal=inp.workload.causal, batch_subset=batch_subset)


FP8_SHAPES = [
    (1, 128, 1, False, [1, 63, 64, 65, 200, 1000]),
    (1, 64, 1, False, [130, 7, 777]),
    (1, 48, 1, False, [5, 300]),
    (2, 64, 1, True, [90, 700, 3]),
    (8, 16, 1, True, [9, 640]),
    (1, 128, 2, False, [100, 257]),
    (1, 16, 1, False, [0, 37, 0, 130]),
]


@pytest.mark.parametrize("s_q,h_q,h_kv,causal,seqlens", FP8_SHAPES)
def test_fp8_decode_shapes(s_q, h_q, h_kv, causal, seqlens):
    inp = _custom(s_q, h_q, h_kv, causal, seqlens, seed=sum(seqlens) + 3)
    o, lse, _ = _run(inp)
    O, LSE = _oracle(inp)
    compare(o, lse, O, LSE, label=f"fp8 {s_q}x{h_q}/{h_kv} causal={causal} L={seqlens}")


@pytest.mark.parametrize("W", [1, 17, 300])
def test_fp8_decode_worker_counts(W):
    inp = _custom(1, 128, 1, False, [70, 1300, 5], seed=W)
    o, lse, _ = _run(inp, num_workers=W)
    O, LSE = _oracle(inp)
    compare(o, lse, O, LSE, label=f"fp8 W={W}")


def test_fp8_poisoned_slots_change_nothing():
    lens = [37, 130, 64, 1]
    clean = _custom(1, 128, 1, False, lens, 3, extra_pages=3)
    dirty = _custom(1, 128, 1, False, lens, 3, extra_pages=3, poison=True)
    assert (dirty.kvcache.numpy() == 0x7F).any()
    a, b = _run(clean), _run(dirty)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_rejects_wide_heads():
    inp = _custom(2, 128, 1, True, [70], seed=1)       # 256 query rows per head
    q, kv, bt, L = (inp.q.to(DEV), inp.kvcache.to(DEV), inp.block_table.to(DEV), inp.cache_seqlens.to(DEV))
    meta, ns = get_mla_metadata(L, 256, 1)
    with pytest.raises(MlaError) as err:
        mla_decode_paged_fp8(q, kv, 0.5, bt, L, 512, meta, ns, causal=True)
    assert err.value.status == -2


@pytest.mark.parametrize("name,k", [("mem_bound", 3), ("skewed", 3)])
def test_fp8_full_size_sampled(name, k):
    inp = make_fp8_inputs(name, 0, encode=oracle_fp8_codes)
    o, lse, splits = _run(inp)
    L = inp.cache_seqlens.numpy()
    picks = sorted(set(np.random.default_rng(1).choice(len(L), size=k, replace=False).tolist())
                   | {int(np.argmax(L)), int(np.argmin(L))})
    O, LSE = _oracle(inp, batch_subset=picks)
    compare(o, lse, O, LSE, batch_subset=picks, label=f"fp8 {name}")


@pytest.mark.parametrize("h_kv,s_new,seqlens", [(1, 1, [0, 1, 63, 64, 65, 127, 128, 4000]),
                                                (2, 3, [5, 62, 200]),
                                                (1, 70, [0, 10, 64])])
def test_fp8_append_bit_exact(h_kv, s_new, seqlens):
    w = Workload("custom", batch=len(seqlens), s_q=1, h_q=16 * h_kv, h_kv=h_kv, causal=False,
                 seqlens=tuple(seqlens), num_pages=None)
    inp, kv_new = make_append_inputs(w, 5, s_new, seqlens=seqlens, extra_pages=2)
    # large values (clamped to +-448 after scaling) and a NaN among the new rows
    kv_new = kv_new.float()
    kv_new[0, 0, 0, :8] = torch.tensor([1e4, -1e4, 200.0, -7.5, float("nan"), 0.0, -0.0, 3e-5])
    kv_new = kv_new.to(torch.bfloat16)
    scale = 1.0 / 64
    P = inp.kvcache.shape[0]
    rng = np.random.default_rng(9)
    before = rng.integers(0, 256, size=(P, 64, h_kv, 576), dtype=np.uint8)
    L = inp.cache_seqlens.numpy().copy()
    bt = inp.block_table.numpy().copy()
    bt[-1, (int(L[-1]) + s_new - 1) // 64] = P + 3            # one row without a valid page
    want, bad = mo.kvcache_append_fp8_ref(before, bt, L, kv_new, np.float32(1.0) / np.float32(scale))
    kv = torch.from_numpy(before).to(DEV)
    bad_rows = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvcache_append_fp8(kv_new.to(DEV), kv, scale, torch.from_numpy(bt).to(DEV), torch.from_numpy(L).to(DEV), bad_rows)
    torch.cuda.synchronize()
    got = kv.cpu().numpy()
    assert int(bad_rows.item()) == bad and bad >= 1
    diff = np.argwhere(got != want)
    assert diff.size == 0, f"{len(diff)} codes differ, first at {diff[0].tolist()}: {got[tuple(diff[0])]} vs {want[tuple(diff[0])]}"


def test_fp8_append_then_decode_end_to_end():
    """bf16 latents appended into an empty fp8 cache on the GPU (three
    sequences, 150 tokens each, over three pages), then decoded from it: the
    codes equal the oracle's append of the same latents bit for bit, and the
    decode matches the oracle's decode of its own cache."""
    scale = 1.0 / 64
    w = Workload("custom", batch=3, s_q=1, h_q=64, h_kv=1, causal=False, seqlens=(0, 0, 0), num_pages=None)
    inp, kv_new = make_append_inputs(w, 21, 150, seqlens=[0, 0, 0], extra_pages=1)
    P = inp.kvcache.shape[0]
    L0 = inp.cache_seqlens.numpy().copy()
    bt = inp.block_table.numpy().copy()
    want, bad = mo.kvcache_append_fp8_ref(np.zeros((P, 64, 1, 576), dtype=np.uint8), bt, L0, kv_new,
                                          np.float32(1.0) / np.float32(scale))
    assert bad == 0
    kv = torch.zeros((P, 64, 1, 576), dtype=torch.uint8, device=DEV)
    bt_d = torch.from_numpy(bt).to(DEV)
    bad_rows = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvcache_append_fp8(kv_new.to(DEV), kv, scale, bt_d, torch.from_numpy(L0).to(DEV), bad_rows)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), want) and int(bad_rows.item()) == 0
    L = torch.from_numpy((L0 + 150).astype(np.int32))
    meta, ns = get_mla_metadata(L.to(DEV), 64, 1)
    o, lse = mla_decode_paged_fp8(inp.q.to(DEV), kv, scale, bt_d, L.to(DEV), 512, meta, ns)
    torch.cuda.synchronize()
    O, LSE = mo.mla_decode_fp8_ref(inp.q, want, scale, bt, L.numpy(), 512)
    compare(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), O, LSE, label="fp8 append then decode")


def test_fp8_one_token_returns_every_code_exactly():
    """A sequence of one token gives that token's value row as O, with weight
    exactly 1: at kv_scale 1 every output element is the E4M3 value of its
    code, which bf16 holds exactly.  The row carries all 254 finite codes
    (twice over the 512 columns), so the decode's code-to-bf16 conversion is
    checked bit for bit against the format's definition."""
    inp = _custom(1, 16, 1, False, [1, 1], seed=3)
    kv = inp.kvcache.clone()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] * 3, dtype=np.uint8)[:512]
    bt = inp.block_table.numpy()
    for b in range(2):
        kv[int(bt[b, 0]), 0, 0, :512] = torch.from_numpy(np.roll(codes, 37 * b))
    inp.kvcache = kv
    inp.extra["kv_scale"] = 1.0
    o, lse, _ = _run(inp)
    for b in range(2):
        want = mo.fp8_e4m3_decode_ref(np.roll(codes, 37 * b))
        got = o[b, 0]                                   # [h_q][512]
        assert np.array_equal(got, np.broadcast_to(want, got.shape)), (b, np.abs(got - want).max())
    O, LSE = _oracle(inp)
    np.testing.assert_allclose(lse, LSE, atol=1e-3)

