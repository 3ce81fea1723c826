"""CPU reference of the split-KV tile scheduler's rule.

TEST INFRASTRUCTURE ONLY (see ``mla_oracle``'s header): the HIP scheduler is
checked against it bit for bit; the library never calls it.

The pages name the call and its outputs -- ``get_mla_metadata(cache_seqlens,
s_q*h_q//h_kv, h_kv)`` returns ``tile_scheduler_metadata, num_splits``
(dolphin-ai.jp FlashMLA page, "FlashMLA の使用方法", step 3) -- and say that a
split-KV kernel runs the pieces and a combine kernel merges them
(deepseek.csdn.net article, section 4.2(1)) with dynamic load balancing over
variable-length sequences (section 4.2(2)).  They give no rule.  This is the
build's own rule ("rule v1"), written as plain loops:

* n_b = ceil(L_b / 64) pages for sequence b.
* A cost line holds, for each sequence in order, H = floor(F / 2) overhead
  units (its query load), its n_b page units, then F - H overhead units (its
  output write).  T = sum_b (F + n_b) and the quota is Q = max(1, ceil(T / W))
  for W workers.  Splitting F around the pages charges each of two workers
  that share a sequence one of the two fixed costs, both of which every
  split pays.
* Worker w owns cost units [w*Q, (w+1)*Q).  Its segments are the
  intersections of that range with each sequence's page units; overhead-only
  intersections give no segment.
* num_splits[0] = 0, num_splits[b+1] = num_splits[b] + (number of workers whose
  range meets b's page units).  Split k of sequence b uses partial slot
  num_splits[b] + k.
* Metadata row w = (begin_b, begin_page, end_b, end_page_exclusive,
  ordinal of the first segment among b's splits, 0, 0, 0).  A worker with no
  segment gets (0, 0, -1, 0, 0, 0, 0, 0).  Only a worker's first segment can
  start inside a sequence, so its later segments have ordinal 0.

W = max(1, N_CU // (h_kv * ceil(R / rb))) for R = s_q*h_q/h_kv query rows per
latent head, with rb = 64 query rows per workgroup for R <= 128 and 128 above.
"""
from __future__ import annotations

import numpy as np

PAGE_SIZE = 64
FIXED_OVERHEAD_PAGES = 2   # F: cost of one sequence's q load and output, in page units
ROWS_PER_BLOCK = 64          # query rows per workgroup for R <= 128 ...
ROWS_PER_WIDE_BLOCK = 128    # ... and for R > 128
METADATA_INTS = 8


def num_workers_ref(n_cu: int, rows_per_kv: int, h_kv: int) -> int:
    rb = ROWS_PER_BLOCK if rows_per_kv <= ROWS_PER_WIDE_BLOCK else ROWS_PER_WIDE_BLOCK
    row_blocks = (rows_per_kv + rb - 1) // rb
    return max(1, n_cu // (h_kv * row_blocks))


def split_rule(cache_seqlens, num_workers: int, fixed_overhead: int = FIXED_OVERHEAD_PAGES):
    """Returns (tile_scheduler_metadata int32 [W][8], num_splits int32 [B+1])."""
    L = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    B, W, F = len(L), int(num_workers), int(fixed_overhead)
    H = F // 2          # overhead units before a sequence's pages; F - H follow them
    n = [(x + PAGE_SIZE - 1) // PAGE_SIZE for x in L]
    start = []          # first page unit of each sequence on the cost line
    pos = 0
    for b in range(B):
        start.append(pos + H)
        pos += F + n[b]
    T = pos
    Q = max(1, -(-T // W))

    num_splits = [0] * (B + 1)
    for b in range(B):
        count = 0
        for w in range(W):
            lo, hi = w * Q, (w + 1) * Q
            if n[b] > 0 and max(lo, start[b]) < min(hi, start[b] + n[b]):
                count += 1
        num_splits[b + 1] = num_splits[b] + count

    meta = [[0, 0, -1, 0, 0, 0, 0, 0] for _ in range(W)]
    for w in range(W):
        lo, hi = w * Q, (w + 1) * Q
        segs = []
        for b in range(B):
            a, e = max(lo, start[b]), min(hi, start[b] + n[b])
            if n[b] > 0 and a < e:
                segs.append((b, a - start[b], e - start[b]))
        if not segs:
            continue
        b0, p0, _ = segs[0]
        b1, _, p1 = segs[-1]
        # ordinal of this worker among the workers meeting sequence b0
        ordinal = 0
        for v in range(w):
            if max(v * Q, start[b0]) < min((v + 1) * Q, start[b0] + n[b0]):
                ordinal += 1
        meta[w] = [b0, p0, b1, p1, ordinal, 0, 0, 0]
    return np.asarray(meta, dtype=np.int32).reshape(W, METADATA_INTS), np.asarray(num_splits, dtype=np.int32)


def segments_of(meta_row, cache_seqlens, num_splits):
    """Expand one metadata row into (b, page_begin, page_end, split_slot) segments."""
    b0, p0, b1, p1, ordinal = (int(x) for x in meta_row[:5])
    out = []
    for b in range(b0, b1 + 1):
        n_b = (int(cache_seqlens[b]) + PAGE_SIZE - 1) // PAGE_SIZE
        lo = p0 if b == b0 else 0
        hi = p1 if b == b1 else n_b
        if hi > lo:
            out.append((b, lo, hi, int(num_splits[b]) + (ordinal if b == b0 else 0)))
    return out
