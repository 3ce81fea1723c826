"""Shared pieces of the GPU tests: run the HIP path through the C ABI on
seeded inputs, and compare with the CPU oracle.

Tolerances for bf16 inputs drawn from N(0, 1): max|dO| <= 1e-2,
mean|dO| <= 1e-3, max|dLSE| <= 1e-3 (O is rounded once to bf16 at the end;
the kernel computes in fp32 with bf16 softmax weights)."""
from __future__ import annotations

import numpy as np
import torch

from oracle.mla_oracle import mla_decode_ref
from paged_mla_decode_03_amd import get_mla_metadata, mla_decode_paged

MAX_ABS_O = 1e-2
MEAN_ABS_O = 1e-3
MAX_ABS_LSE = 1e-3

DEV = torch.device("cuda", 0)


def to_dev(inp):
    return (inp.q.to(DEV), inp.kvcache.to(DEV), inp.block_table.to(DEV), inp.cache_seqlens.to(DEV))


def run_gpu(inp, causal=None, num_workers=None, softmax_scale=None, dev_tensors=None):
    """One decode step on the GPU; returns host (o fp64, lse fp64, meta, num_splits)."""
    w = inp.workload
    q, kv, bt, L = dev_tensors or to_dev(inp)
    causal = w.causal if causal is None else causal
    meta, ns = get_mla_metadata(L, w.s_q * w.h_q // w.h_kv, w.h_kv, num_workers)
    o, lse = mla_decode_paged(q, kv, bt, L, 512, meta, ns, causal=causal, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return (o.float().cpu().double().numpy(), lse.cpu().double().numpy(), meta.cpu().numpy(), ns.cpu().numpy())


def oracle(inp, causal=None, batch_subset=None, softmax_scale=None):
    w = inp.workload
    causal = w.causal if causal is None else causal
    return mla_decode_ref(inp.q, inp.kvcache, inp.block_table.numpy(), inp.cache_seqlens.numpy(), 512,
                          causal=causal, softmax_scale=softmax_scale, batch_subset=batch_subset)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


def compare(o, lse, O, LSE, batch_subset=None, scale=1.0, ulp_aware=False, label=""):
    """Assert the GPU result (o, lse) matches the oracle (O, LSE) on the
    sequences in batch_subset (all when None).  `scale` widens the O bars for
    inputs whose values are larger than N(0, 1).  With `ulp_aware`, an output
    element may also differ by one bf16 ulp of its exact value plus 2e-3 (the
    kernel's error before the final rounding, which may round to the far
    neighbour): where |O| approaches 4 (rows that average one to three cached
    values) the final bf16 rounding alone exceeds 1e-2."""
    idx = slice(None) if batch_subset is None else np.asarray(batch_subset)
    o, O, lse, LSE = o[idx], O[idx], lse[idx], LSE[idx]
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    d = np.abs(o - O)
    if ulp_aware:
        d = np.where(d <= bf16_ulp(O) + 2e-3, 0.0, d)
    neg = np.isneginf(LSE)
    assert (np.isneginf(lse) == neg).all(), f"{label}: -inf LSE pattern differs"
    dl = np.abs(lse[~neg] - LSE[~neg]) if (~neg).any() else np.zeros(1)
    stats = dict(max_o=float(d.max()), mean_o=float(d.mean()), max_lse=float(dl.max()))
    assert stats["max_o"] <= MAX_ABS_O * scale, f"{label}: {stats}"
    assert stats["mean_o"] <= MEAN_ABS_O * scale, f"{label}: {stats}"
    assert stats["max_lse"] <= MAX_ABS_LSE, f"{label}: {stats}"
    return stats
