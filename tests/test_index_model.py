"""Host model of the decode path's indexing, checked against the extents of
the buffers the library is handed.

For given inputs it walks what every workgroup of the decode touches, in the
kernels' own order: the worker's segments (metadata from the split-rule
reference), the load cursor that runs up to three half pages (64-row
kernel) or one page (128-row kernel) ahead across segment ends, the order of
a segment's pages in each row block, the block_table entries it reads, the
page ids it builds DMA resources from (an id outside the pool gets a
resource of size 0, so no address outside the cache is formed), the partial
slots it writes and the combine's reads of them, and the output and lse
elements.  Every index must lie inside its allocation:

  block_table [B][max_pages], page pool [num_pages], split partials
  [W + B][h_kv][R] (+ 512 columns), o [B][s_q][h_q][512], lse [B][h_q][s_q].

Run on the tiny workload's exact inputs (seeds 0-2, a pool of 8 pages with
4 unreferenced) and on every parity shape and measured workload, it shows
the current indexing clean on the CPU for the input that faulted the GPU
with an earlier kernel.  It is a model of the index arithmetic, not an
execution of the kernel source."""
import numpy as np
import pytest

from oracle import sched_ref
from workloads import WORKLOADS, Workload, make_inputs

PAGE = 64
N_CU = 256


def _pages_of(L):
    return (L + PAGE - 1) // PAGE if L > 0 else 0


def _page_in_order(page, p0, end, rb, nrb):
    """Page that step `page` of segment [p0, end) processes in row block rb."""
    j = page - p0 - 1
    if j < 0 or nrb == 1:
        return page
    base = p0 + 1 + (j // nrb) * nrb
    if base + nrb > end:
        return page
    r = j - (j // nrb) * nrb + rb
    return base + (r - nrb if r >= nrb else r)


class Extents:
    """Records every index and checks it against its buffer."""

    def __init__(self, B, max_pages, num_pages, W, h_kv, R, s_q, h_q):
        self.lim = dict(table=B * max_pages, ws_o=(W + B) * h_kv * R * 512, ws_lse=(W + B) * h_kv * R,
                        o=B * s_q * h_q * 512, lse=B * h_q * s_q)
        self.num_pages = num_pages
        self.touched = {k: 0 for k in self.lim}
        self.dma_pages = set()

    def use(self, buf, idx):
        assert 0 <= idx < self.lim[buf], f"{buf}[{idx}] outside [0, {self.lim[buf]})"
        self.touched[buf] += 1


def walk(bt, L, s_q, h_q, h_kv, causal=False, num_workers=None):
    """Model one decode launch (decode, then combine); returns the extents record."""
    bt = np.asarray(bt)
    L = [int(x) for x in L]
    B, max_pages = bt.shape
    num_pages = int(bt.max()) + 1 if bt.size else 1
    R = s_q * (h_q // h_kv)
    group = h_q // h_kv
    rows_per_block = 64 if R <= 128 else 128
    nrb = -(-R // rows_per_block)
    W = num_workers or sched_ref.num_workers_ref(N_CU, R, h_kv)
    meta, ns = sched_ref.split_rule(L, W)
    ext = Extents(B, max_pages, num_pages, W, h_kv, R, s_q, h_q)
    lookahead_pages = 2 if rows_per_block == 64 else 1   # 3 half pages ahead = into the second next page

    def page_id(b, j):
        if j >= max_pages:                      # past the table row: -1, nothing read
            return -1
        ext.use("table", b * max_pages + j)
        return int(bt[b, j])

    for w in range(W):
        segs = sched_ref.segments_of(meta[w], L, ns)
        if int(meta[w][2]) < int(meta[w][0]) or not segs:
            continue
        for g in range(h_kv):
            for rb in range(nrb):
                # the worker's pages in load order, as the load cursor visits them
                order = []
                for b, lo, hi, slot in segs:
                    assert 0 <= lo < hi <= _pages_of(L[b])
                    order += [(b, _page_in_order(pg, lo, hi, rb, nrb)) for pg in range(lo, hi)]
                # the load cursor stops at the worker's last page; the steps
                # before it look ahead, never past it
                for step in range(len(order)):
                    for ahead in range(lookahead_pages + 1):
                        if step + ahead < len(order):
                            b, j = order[step + ahead]
                            pid = page_id(b, j)
                            if 0 <= pid < num_pages:
                                ext.dma_pages.add(pid)
                # outputs of each segment
                for b, lo, hi, slot in segs:
                    nsplit = int(ns[b + 1] - ns[b])
                    assert int(ns[b]) <= slot < int(ns[b + 1]) <= W + B
                    for r in range(rows_per_block):
                        qrow = rb * rows_per_block + r
                        if qrow >= R:
                            continue
                        tok, head = qrow // group, g * group + qrow % group
                        if nsplit == 1:
                            ext.use("o", ((b * s_q + tok) * h_q + head) * 512 + 511)
                            ext.use("lse", (b * h_q + head) * s_q + tok)
                        else:
                            ext.use("ws_o", ((slot * h_kv + g) * R + qrow) * 512 + 511)
                            ext.use("ws_lse", (slot * h_kv + g) * R + qrow)
    # combine: every split sequence reads its slots and writes o and lse
    for b in range(B):
        n = int(ns[b + 1] - ns[b])
        if n <= 1:
            continue
        for s in range(int(ns[b]), int(ns[b + 1])):
            for g in range(h_kv):
                ext.use("ws_lse", (s * h_kv + g) * R + R - 1)
                ext.use("ws_o", ((s * h_kv + g) * R + R - 1) * 512 + 511)
        ext.use("o", ((b * s_q + s_q - 1) * h_q + h_q - 1) * 512 + 511)
        ext.use("lse", (b * h_q + h_q - 1) * s_q + s_q - 1)
    # every referenced page was staged, and only referenced pages
    ref = {int(bt[b, j]) for b in range(B) for j in range(_pages_of(L[b]))}
    assert ext.dma_pages == ref, (sorted(ext.dma_pages), sorted(ref))
    return ext


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_inputs_index_clean(seed):
    inp = make_inputs("tiny", seed)
    w = inp.workload
    bt = inp.block_table.numpy()
    assert inp.kvcache.shape[0] == 8                       # the 8-page pool
    ext = walk(bt, inp.cache_seqlens.numpy(), w.s_q, w.h_q, w.h_kv, w.causal)
    assert bt.max() < 8 and len(ext.dma_pages) == 4        # four pages referenced, four never staged
    for W in (1, 3, 17, 300):                              # user-chosen worker counts too
        walk(bt, inp.cache_seqlens.numpy(), w.s_q, w.h_q, w.h_kv, w.causal, num_workers=W)


SHAPES = [(1, 16, 1, [0, 37, 0, 130]), (1, 128, 1, [1, 63, 64, 65, 200, 1000]), (2, 64, 1, [90, 700, 3]),
          (8, 16, 1, [9, 640]), (1, 128, 2, [100, 257]), (2, 128, 1, [70, 5000]), (4, 128, 1, [1, 129])]


@pytest.mark.parametrize("s_q,h_q,h_kv,seqlens", SHAPES)
def test_parity_shapes_index_clean(s_q, h_q, h_kv, seqlens):
    w = Workload("custom", batch=len(seqlens), s_q=s_q, h_q=h_q, h_kv=h_kv, causal=False,
                 seqlens=tuple(seqlens), num_pages=None)
    inp = make_inputs(w, 1, seqlens=seqlens)
    walk(inp.block_table.numpy(), inp.cache_seqlens.numpy(), s_q, h_q, h_kv)


@pytest.mark.parametrize("name", ["mem_bound", "var_len", "causal_sq2", "skewed"])
def test_workloads_index_clean(name):
    inp = make_inputs(name, 0)
    w = inp.workload
    walk(inp.block_table.numpy(), inp.cache_seqlens.numpy(), w.s_q, w.h_q, w.h_kv, w.causal)


def test_model_sees_planted_index_mistakes(monkeypatch):
    """An off-by-one in the page order (a step one page too far) and a slot
    one past the partials both fail."""
    inp = make_inputs("tiny", 0)
    w = inp.workload
    monkeypatch.setattr(__import__(__name__), "_page_in_order",
                        lambda page, p0, end, rb, nrb: page + 1)
    with pytest.raises((AssertionError, IndexError)):
        walk(inp.block_table.numpy(), inp.cache_seqlens.numpy(), w.s_q, w.h_q, w.h_kv)
    bad = Extents(2, 3, 6, 1, 1, 16, 1, 16)
    with pytest.raises(AssertionError):
        bad.use("ws_lse", (1 + 2) * 16)                     # one past the last slot
    with pytest.raises(AssertionError):
        bad.use("table", 2 * 3)                             # one past the table
