"""Seeded synthetic inputs for paged MLA decode.

This module only draws inputs: sequence lengths, the page permutation behind
``block_table``, and bf16 values for ``q`` and the latent KV cache. It holds none
of the attention arithmetic, so both the CPU oracle (``oracle/``) and the HIP
library's tests and benchmark can take their inputs from it without sharing any
part of the method.

Layouts (the paged-cache contract of the deepseek.csdn.net FlashMLA article,
section 4.2(1) "Paged KV Cache": 64-token blocks, ``block_table`` maps a
sequence's logical block to a physical page):

* ``q``            bf16 ``[B][s_q][h_q][576]``  absorbed query rows [q^C-absorbed (512); q^R (64)]
* ``kvcache``      bf16 ``[num_pages][64][h_kv][576]``  cached row [c^KV (512); k^R (64)]
* ``block_table``  int32 ``[B][max_pages_per_seq]``  physical page of logical block j; padding -1
* ``cache_seqlens`` int32 ``[B]``

Recipe: numpy ``Generator(PCG64(seed))``; draw order is sequence lengths (when
random), then the page permutation, then ``q``, then ``kvcache``.  Values are
float32 ``standard_normal`` rounded to bf16 (round-to-nearest-even, done by
torch on the host), so every consumer sees identical bytes.  Block-table rows
take consecutive chunks of ``rng.permutation(num_pages)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np
import torch

PAGE_SIZE = 64
D_QK = 576
D_V = 512


@dataclass(frozen=True)
class Workload:
    """Shape of one decode step.  ``seqlens`` is a fixed list, or ``None`` when
    ``seqlen_rule`` draws it from the seed."""

    name: str
    batch: int
    s_q: int
    h_q: int
    h_kv: int
    causal: bool
    seqlens: Optional[tuple] = None
    seqlen_rule: str = "fixed"        # fixed | loguniform | skewed
    seqlen_max: int = 0               # loguniform upper bound
    long_len: int = 0                 # skewed: the one long sequence
    short_range: tuple = (0, 0)       # skewed: inclusive range of the others
    num_pages: Optional[int] = None   # pool size; None = exactly the pages used
    d_qk: int = D_QK
    d_v: int = D_V
    description: str = ""

    @property
    def rows_per_kv(self) -> int:
        return self.s_q * self.h_q // self.h_kv


# The five workloads the build is measured and checked on.
WORKLOADS = {
    "tiny": Workload(
        "tiny", batch=2, s_q=1, h_q=16, h_kv=1, causal=False, seqlens=(37, 130), num_pages=8,
        description="B=2, s_q=1, h_q=16, L={37,130}, pool of 8 pages"),
    "mem_bound": Workload(
        "mem_bound", batch=64, s_q=1, h_q=128, h_kv=1, causal=False, seqlens=(4096,) * 64,
        num_pages=4096,
        description="B=64, s_q=1, h_q=128, every L=4096, pool of 4096 pages"),
    "var_len": Workload(
        "var_len", batch=128, s_q=1, h_q=128, h_kv=1, causal=False, seqlen_rule="loguniform",
        seqlen_max=16384,
        description="B=128, s_q=1, h_q=128, L log-uniform in [1,16384]"),
    "causal_sq2": Workload(
        "causal_sq2", batch=132, s_q=2, h_q=128, h_kv=1, causal=True, seqlens=(8192,) * 132,
        description="B=132, s_q=2 causal, h_q=128, every L=8192"),
    "skewed": Workload(
        "skewed", batch=16, s_q=1, h_q=128, h_kv=1, causal=False, seqlen_rule="skewed",
        long_len=131072, short_range=(512, 2048),
        description="B=16, s_q=1, h_q=128, one L=131072, others U[512,2048]"),
}


def draw_seqlens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """Sequence lengths for ``w`` (consumes the generator only for random rules)."""
    if w.seqlen_rule == "fixed":
        assert w.seqlens is not None and len(w.seqlens) == w.batch
        return np.asarray(w.seqlens, dtype=np.int64)
    if w.seqlen_rule == "loguniform":
        u = rng.uniform(0.0, math.log(w.seqlen_max), size=w.batch)
        return np.clip(np.rint(np.exp(u)), 1, w.seqlen_max).astype(np.int64)
    if w.seqlen_rule == "skewed":
        long_idx = int(rng.integers(w.batch))
        lo, hi = w.short_range
        short = rng.integers(lo, hi, size=w.batch - 1, endpoint=True)
        out = np.empty(w.batch, dtype=np.int64)
        out[np.arange(w.batch) != long_idx] = short
        out[long_idx] = w.long_len
        return out
    raise ValueError(f"unknown seqlen rule {w.seqlen_rule!r}")


def bf16_normal(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> torch.Tensor:
    """float32 standard normals rounded to bf16 (RNE), drawn in order, in chunks
    so that a 1.2 GB cache does not need a 5 GB float64 temporary."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = torch.from_numpy(rng.standard_normal(e - s, dtype=np.float32)).to(torch.bfloat16)
    return out.view(*shape)


@dataclass
class DecodeInputs:
    workload: Workload
    seed: int
    q: torch.Tensor               # bf16 [B][s_q][h_q][576]
    kvcache: torch.Tensor         # bf16 [P][64][h_kv][576]
    block_table: torch.Tensor     # int32 [B][max_pages]
    cache_seqlens: torch.Tensor   # int32 [B]
    extra: dict = field(default_factory=dict)

    @property
    def pages_per_seq(self) -> np.ndarray:
        return (self.cache_seqlens.numpy().astype(np.int64) + PAGE_SIZE - 1) // PAGE_SIZE


def make_inputs(w: Workload | str, seed: int = 0, *, seqlens=None, poison: bool = False,
                max_pages_per_seq: Optional[int] = None, extra_pages: int = 0) -> DecodeInputs:
    """Draw one decode step's inputs.

    ``seqlens`` overrides the workload's lengths (the generator still draws the
    page permutation, then q, then the cache).  ``poison`` writes NaN into every
    cache slot no sequence may read (tail slots of each last page, pages of the
    pool that no block-table row uses); block-table padding is always -1.
    ``extra_pages`` enlarges the pool with pages nobody references."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.Generator(np.random.PCG64(seed))
    if seqlens is None:
        L = draw_seqlens(w, rng)
    else:
        L = np.asarray(seqlens, dtype=np.int64)
        w = replace(w, batch=len(L), seqlens=tuple(int(x) for x in L), seqlen_rule="fixed")
    n_pages = (L + PAGE_SIZE - 1) // PAGE_SIZE
    used = int(n_pages.sum())
    pool = w.num_pages if (w.num_pages is not None and seqlens is None) else used
    pool = max(pool, used) + extra_pages
    mp = int(n_pages.max()) if len(n_pages) else 0
    if max_pages_per_seq is not None:
        assert max_pages_per_seq >= mp
        mp = max_pages_per_seq
    mp = max(mp, 1)
    perm = rng.permutation(pool)
    bt = np.full((w.batch, mp), -1, dtype=np.int32)
    off = 0
    for b in range(w.batch):
        bt[b, : n_pages[b]] = perm[off: off + n_pages[b]]
        off += int(n_pages[b])
    q = bf16_normal(rng, (w.batch, w.s_q, w.h_q, w.d_qk))
    kv = bf16_normal(rng, (pool, PAGE_SIZE, w.h_kv, w.d_qk))
    if poison:
        nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
        referenced = np.zeros(pool, dtype=bool)
        for b in range(w.batch):
            pages = bt[b, : n_pages[b]]
            referenced[pages] = True
            tail = int(L[b]) % PAGE_SIZE
            if n_pages[b] > 0 and tail:
                kv[int(pages[-1]), tail:] = nan
        kv[torch.from_numpy(~referenced)] = nan
    return DecodeInputs(w, seed, q, kv, torch.from_numpy(bt), torch.from_numpy(L.astype(np.int32)))


def make_append_inputs(w: Workload | str, seed: int = 0, s_new: int = 1, *, seqlens=None,
                       extra_pages: int = 0):
    """Inputs of a cache append: the workload's lengths L (or ``seqlens``)
    are drawn as for a decode step, the block table maps pages for L + s_new
    tokens, and ``cache_seqlens`` holds L (the tokens cached before the
    append).  Returns (inputs, kv_new bf16 [B][s_new][h_kv][576])."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if seqlens is None:
        seqlens = draw_seqlens(w, np.random.Generator(np.random.PCG64(seed)))
    L = np.asarray(seqlens, dtype=np.int64)
    inp = make_inputs(w, seed, seqlens=L + s_new, extra_pages=extra_pages)
    inp.cache_seqlens = torch.from_numpy(L.astype(np.int32))
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    kv_new = bf16_normal(rng, (len(L), s_new, w.h_kv, w.d_qk))
    return inp, kv_new


def algorithmic_counts(w: Workload, seqlens: np.ndarray, max_pages_per_seq: int) -> dict:
    """Bytes and flops one decode step needs by definition: every visible latent
    row read once (h_kv * 576 bf16 per token), q read once, o and lse written
    once, the block table and seqlens read once; two multiply-adds per
    (query row, visible key, output column) for the 576-wide scores and the
    512-wide weighted sum.  Masked pairs, tail slots, split partials and
    re-reads are implementation costs and are not counted."""
    L = np.asarray(seqlens, dtype=np.int64)
    B = len(L)
    kv_bytes = int(L.sum()) * w.h_kv * w.d_qk * 2
    q_bytes = B * w.s_q * w.h_q * w.d_qk * 2
    o_bytes = B * w.s_q * w.h_q * w.d_v * 2
    lse_bytes = B * w.h_q * w.s_q * 4
    table_bytes = B * max_pages_per_seq * 4 + B * 4
    if w.causal:
        vis = sum(int(max(0, min(l, l - w.s_q + i + 1))) for l in L for i in range(w.s_q))
    else:
        vis = int(L.sum()) * w.s_q
    flops = 2 * vis * w.h_q * (w.d_qk + w.d_v)
    return dict(kv_bytes=kv_bytes, total_bytes=kv_bytes + q_bytes + o_bytes + lse_bytes + table_bytes,
                flops=flops, visible_pairs_per_head=vis)


# fp8 cache inputs: one byte per cached value (OCP FP8 E4M3 codes) and one
# scale for the whole cache.  The cache holds what a quantising append leaves
# for the workload's N(0, 1) latents: with the scale 1/64 a latent of
# magnitude up to 7 maps into the format's range (+-448), so the codes of
# normal data are never clamped and sit in the format's upper binades, as a
# scale fitted to the latents' range puts them.
FP8_KV_SCALE = 1.0 / 64.0


def make_fp8_inputs(w: Workload | str, seed: int = 0, *, encode, seqlens=None, poison: bool = False,
                    extra_pages: int = 0) -> DecodeInputs:
    """A decode step over an fp8 cache: the lengths, block table, q and bf16
    latents of :func:`make_inputs` (same draws), with the cache replaced by
    ``encode(latents, kv_scale)``: the caller's quantiser, returning uint8
    codes [P][64][h_kv][576] of latents / kv_scale.  ``poison`` puts the NaN
    code 0x7F into every slot no sequence may read.  The scale is in
    ``extra["kv_scale"]``."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    base = make_inputs(w, seed, seqlens=seqlens, extra_pages=extra_pages)
    shape = tuple(base.kvcache.shape)
    codes = np.ascontiguousarray(np.asarray(encode(base.kvcache, FP8_KV_SCALE), dtype=np.uint8))
    if codes.shape != shape:
        raise ValueError(f"encoder returned shape {codes.shape}, expected {shape}")
    if poison:
        L = base.cache_seqlens.numpy()
        bt = base.block_table.numpy()
        referenced = np.zeros(shape[0], dtype=bool)
        for b in range(len(L)):
            npg = (int(L[b]) + PAGE_SIZE - 1) // PAGE_SIZE
            pages = bt[b, :npg]
            referenced[pages] = True
            tail = int(L[b]) % PAGE_SIZE
            if npg > 0 and tail:
                codes[int(pages[-1]), tail:] = 0x7F
        codes[~referenced] = 0x7F
    base.kvcache = torch.from_numpy(codes)
    base.extra["kv_scale"] = FP8_KV_SCALE
    return base
