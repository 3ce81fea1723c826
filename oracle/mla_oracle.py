"""CPU fp64 oracle for paged Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it and shares no code with it.

What it computes (deepseek.csdn.net, "FlashMLA ... 详解", section 2.2 "DeepSeek-V3
的MLA机制"):

* The output equation of that section: for query token t and head i,
  o_{t,i} = sum_{j<=t} Softmax_j(q_{t,i}^T k_{j,i} / sqrt(d_h + d_h^R)) v_{j,i}.
* The paragraph after it: only c^KV_t and k^R_t are cached; everything else is
  recovered by matrix absorption.  After absorption a query head is one
  576-wide row [W^UK^T q^C (512); q^R (64)], its keys are the cached rows
  [c^KV (512); k^R (64)] (the concatenation order of equations (4) and (9)),
  and its values are the first ``dv`` = 512 columns of the same rows (c^KV),
  so the output stays in latent space.
* The paged cache of section 4.2(1): 64-token blocks, ``block_table`` maps a
  sequence's logical block to its physical page.
* Appending new tokens to the paged cache (:func:`kvcache_append_ref`): the
  cache keeps every earlier token's latent row, and a new token's row goes to
  the page and slot its logical position maps to.
* The output projection over all heads (:func:`out_proj_ref`), the second
  output equation of section 2.2: u_t = W^O [o_{t,1}; ...; o_{t,n_h}].
* Whole-page allocation for the paged cache (:func:`pages_init_ref`,
  :func:`pages_reserve_ref`, :func:`pages_release_ref`): memory is handed
  out and taken back only in whole 64-token pages (the lukefan.com talk on
  FlashMLA, on allocating and freeing in whole pages of 64; the
  deepseek.csdn.net article, section 4.2(2), paged KV cache management).
* An fp8 cache (:func:`fp8_e4m3_encode_ref`, :func:`fp8_e4m3_decode_ref`,
  :func:`kvcache_append_fp8_ref`, :func:`mla_decode_fp8_ref`): the
  ruibaoantu.com page's outlook on mixing BF16 with FP8; read here as a
  cache whose latent rows are stored in fp8 while queries, the arithmetic
  and the outputs stay bf16/fp32.
* The call on the dolphin-ai.jp FlashMLA page ("FlashMLA の使用方法", step 4):
  ``flash_mla_with_kvcache(q, kvcache, block_table, cache_seqlens, dv, ...,
  causal)`` returns the output and the log-sum-exp.

Readings where the pages are silent:

* scale sigma = 1/sqrt(192) by default (d_h = 128, d_h^R = 64);
* LSE = natural log of sum_j exp(sigma * q.k_j), the scale included;
* causal rows are bottom-right aligned: the s_q new tokens are the last s_q
  cache entries, query token i sees keys 0 .. L - s_q + i;
* a row that sees no key returns O = 0, LSE = -inf;
* query head h uses latent head h // (h_q / h_kv).

Layouts: q [B][s_q][h_q][576], kvcache [P][64][h_kv][576], block_table
[B][max_pages], cache_seqlens [B].  Returns O [B][s_q][h_q][dv] and LSE
[B][h_q][s_q], both float64.
"""
from __future__ import annotations

import math

import numpy as np

PAGE_SIZE = 64
DEFAULT_SCALE = 1.0 / math.sqrt(128 + 64)


def as_f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (bf16 included) to float64.
    bf16 -> fp64 is exact."""
    if hasattr(x, "detach"):
        import torch  # only for the dtype conversion of a host tensor

        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def gather_latent_rows(kvcache, block_table_row, seqlen: int, g: int) -> np.ndarray:
    """Rows 0..seqlen-1 of one sequence's latent head g, in logical order, as
    float64: token j lives at page block_table_row[j // 64], slot j % 64.
    Slots at or beyond ``seqlen`` are never read.  ``kvcache`` may be a numpy
    array or a host torch tensor; only the gathered slots are upcast."""
    n_blocks = (seqlen + PAGE_SIZE - 1) // PAGE_SIZE
    rows = np.empty((seqlen, kvcache.shape[-1]), dtype=np.float64)
    for blk in range(n_blocks):
        page = int(block_table_row[blk])
        count = min(PAGE_SIZE, seqlen - blk * PAGE_SIZE)
        rows[blk * PAGE_SIZE: blk * PAGE_SIZE + count] = as_f64(kvcache[page, :count, g, :])
    return rows


def visible_keys(seqlen: int, s_q: int, i: int, causal: bool) -> int:
    """How many leading keys query token i sees (bottom-right causal alignment)."""
    if not causal:
        return seqlen
    return max(0, min(seqlen, seqlen - s_q + i + 1))


def attend(q_rows: np.ndarray, keys: np.ndarray, n_vis, dv: int, scale: float, return_p=False):
    """Softmax attention of each query row r over its first n_vis[r] keys.

    s_j = scale * q.k_j;  LSE = m + ln sum_j exp(s_j - m) with m = max_j s_j;
    p_j = exp(s_j - LSE);  O = sum_j p_j * k_j[0:dv].
    Rows with no visible key give O = 0, LSE = -inf."""
    R = q_rows.shape[0]
    S = scale * (q_rows @ keys.T) if keys.shape[0] else np.zeros((R, 0))
    O = np.zeros((R, dv))
    lse = np.full(R, -np.inf)
    ps = []
    for r in range(R):
        n = int(n_vis[r])
        if n == 0:
            ps.append(np.zeros(0))
            continue
        s = S[r, :n]
        m = s.max()
        lse[r] = m + math.log(np.exp(s - m).sum())
        p = np.exp(s - lse[r])
        O[r] = p @ keys[:n, :dv]
        ps.append(p)
    return (O, lse, ps) if return_p else (O, lse)


def mla_decode_ref(q, kvcache, block_table, cache_seqlens, dv: int = 512, causal: bool = False,
                   softmax_scale: float | None = None, return_p: bool = False, batch_subset=None):
    """Paged MLA decode, by definition, in float64.

    For each sequence b and latent head g: gather the sequence's cached rows
    in logical order, take the s_q * (h_q/h_kv) query rows that share head g,
    and apply :func:`attend` with each row's causal key count.
    ``batch_subset`` restricts the work to some sequences (others stay 0/-inf)."""
    q = as_f64(q)
    bt = np.asarray(block_table)
    L = np.asarray(cache_seqlens).astype(np.int64)
    B, s_q, h_q, D = q.shape
    h_kv = kvcache.shape[2]
    assert kvcache.shape[1] == PAGE_SIZE and kvcache.shape[3] == D and h_q % h_kv == 0
    G = h_q // h_kv
    scale = DEFAULT_SCALE if softmax_scale is None else float(softmax_scale)
    O = np.zeros((B, s_q, h_q, dv))
    LSE = np.full((B, h_q, s_q), -np.inf)
    P = {}
    for b in (range(B) if batch_subset is None else batch_subset):
        for g in range(h_kv):
            keys = gather_latent_rows(kvcache, bt[b], int(L[b]), g)
            rows = q[b, :, g * G:(g + 1) * G, :].reshape(s_q * G, D)
            n_vis = [visible_keys(int(L[b]), s_q, r // G, causal) for r in range(s_q * G)]
            res = attend(rows, keys, n_vis, dv, scale, return_p)
            o_bg, lse_bg = res[0], res[1]
            O[b, :, g * G:(g + 1) * G, :] = o_bg.reshape(s_q, G, dv)
            LSE[b, g * G:(g + 1) * G, :] = lse_bg.reshape(s_q, G).T
            if return_p:
                for r in range(s_q * G):
                    P[(b, r // G, g * G + r % G)] = res[2][r]
    return (O, LSE, P) if return_p else (O, LSE)


def attend_range(q_rows: np.ndarray, keys: np.ndarray, lo: int, hi: int, n_vis, dv: int, scale: float):
    """Attention restricted to keys [lo, hi) (and to each row's visible prefix):
    the normalised partial output and its log-sum-exp, as one split of the key
    range produces them (deepseek.csdn.net article, section 4.2(1): a split-KV
    forward kernel followed by a kernel that merges the splits)."""
    R = q_rows.shape[0]
    vis = [max(0, min(hi, int(n_vis[r])) - lo) for r in range(R)]
    sub = keys[lo:hi]
    return attend(q_rows, sub, vis, dv, scale)


def lse_combine_ref(partial_o: np.ndarray, partial_lse: np.ndarray):
    """Merge n partial results of disjoint key ranges.

    partial_o [n][R][dv] (each normalised by its own sum), partial_lse [n][R].
    lse = M + ln sum_s exp(lse_s - M) with M = max_s lse_s, and
    O = sum_s exp(lse_s - lse) * O_s.  Splits with lse_s = -inf carry no
    weight; if every split is empty the row is O = 0, lse = -inf."""
    n, R, dv = partial_o.shape
    O = np.zeros((R, dv))
    lse = np.full(R, -np.inf)
    for r in range(R):
        ls = partial_lse[:, r]
        M = ls.max() if n else -np.inf
        if not np.isfinite(M):
            continue
        lse[r] = M + math.log(np.exp(ls - M).sum())
        w = np.exp(ls - lse[r])
        O[r] = (w[:, None] * partial_o[:, r, :]).sum(axis=0)
    return O, lse


def kvcache_append_ref(kvcache, block_table, cache_seqlens, kv_new):
    """Write the latent rows of new tokens into the paged cache.

    The cache holds each token's [c^KV; k^R] row once it is computed, so a
    decode step only computes the new token's row and keeps every earlier one
    (deepseek.csdn.net FlashMLA article, section 4.1 on the KV cache); pages
    of 64 slots are mapped through block_table (same article, section
    4.2(1)).  New token i of sequence b
    takes logical position L_b + i, where L_b = cache_seqlens[b] counts the
    tokens cached before the call, i.e. page block_table[b][(L_b + i) // 64],
    slot (L_b + i) % 64.

    kvcache [P][64][h_kv][D] and kv_new [B][s_new][h_kv][D] are arrays of one
    element type (bf16 as uint16 bits, or any numpy dtype): this is a copy,
    so the result is exact.  A row whose position lies past the block
    table (L_b < 0, or (L_b + i) // 64 >= max_pages) or whose page id lies
    outside [0, P) is not written and is counted.  Returns (new cache,
    number of rows not written)."""
    out = np.array(kvcache, copy=True)
    new = np.asarray(kv_new)
    bt = np.asarray(block_table)
    L = np.asarray(cache_seqlens).astype(np.int64)
    B, s_new, h_kv, D = new.shape
    P, page, h_kv2, D2 = out.shape
    assert page == PAGE_SIZE and h_kv2 == h_kv and D2 == D and bt.shape[0] == B and L.shape == (B,)
    max_pages = bt.shape[1]
    bad = 0
    for b in range(B):
        for i in range(s_new):
            pos = int(L[b]) + i
            blk = pos // PAGE_SIZE
            pid = int(bt[b, blk]) if L[b] >= 0 and blk < max_pages else -1
            for g in range(h_kv):
                if not 0 <= pid < P:
                    bad += 1
                    continue
                out[pid, pos % PAGE_SIZE, g, :] = new[b, i, g, :]
    return out, bad


def absorb_q_ref(q_nope, q_rope, w_uk_t):
    """Absorbed query rows (deepseek.csdn.net FlashMLA article, section 2.2,
    the matrix-absorption paragraph): since k^C = W^UK c^KV, the score
    q^C . k^C equals (W^UK^T q^C) . c^KV, so a head's query against the cached
    latent row is [W^UK^T q^C ; q^R].

    q_nope [T][h][128], q_rope [T][h][64], w_uk_t [h][512][128] (W^UK of
    each head stored transposed, c-major).  Returns [T][h][576] in float64."""
    qn, qr, w = as_f64(q_nope), as_f64(q_rope), as_f64(w_uk_t)
    T, H, _ = qn.shape
    out = np.zeros((T, H, w.shape[1] + qr.shape[2]))
    for h in range(H):
        out[:, h, : w.shape[1]] = qn[:, h, :] @ w[h].T
        out[:, h, w.shape[1]:] = qr[:, h, :]
    return out


def absorb_o_ref(o_latent, w_uv):
    """Per-head output from the latent one (same paragraph): v^C = W^UV c^KV,
    and the attention weights sum over the same keys, so sum_j p_j v^C_j =
    W^UV sum_j p_j c^KV_j.

    o_latent [T][h][512], w_uv [h][128][512].  Returns [T][h][128] in float64."""
    o, w = as_f64(o_latent), as_f64(w_uv)
    T, H, _ = o.shape
    out = np.zeros((T, H, w.shape[1]))
    for h in range(H):
        out[:, h, :] = o[:, h, :] @ w[h].T
    return out


def out_proj_ref(o_heads, w_o):
    """The output projection over all heads (deepseek.csdn.net FlashMLA
    article, section 2.2, second output equation): the per-head outputs
    o_{t,i} are stacked in head order, [o_{t,1}; o_{t,2}; ...; o_{t,n_h}],
    and mapped by one matrix, u_t = W^O [o_{t,1}; ...; o_{t,n_h}].

    o_heads [T][h][d_h], w_o [d_model][h * d_h].  Returns [T][d_model] in
    float64."""
    o, w = as_f64(o_heads), as_f64(w_o)
    T, H, D = o.shape
    stacked = o.reshape(T, H * D)          # row t = o_{t,1} followed by o_{t,2}, ...
    return stacked @ w.T


# ----------------------------------------------------------------------------
# Whole-page allocation.
#
# The pool holds num_pages pages of 64 token slots; a sequence's cache is
# always a whole number of pages, mapped through its block_table row.  The
# free pages form a stack: free_pages[0 .. count) with the top at count - 1.
# The order in which pages are handed out is this implementation's own rule
# (the pages only ask for whole pages):
#   * init: free_pages[i] = num_pages - 1 - i, so the first pages handed out
#     are 0, 1, 2, ...;
#   * reserve (before appending s_new tokens to every sequence of lengths L):
#     sequence b needs ceil((L_b + s_new) / 64) - ceil(L_b / 64) more pages;
#     sequences in batch order, and each one's blocks in ascending order, take
#     pages popped from the top of the stack;
#   * release (sequences whose flag is set): each one's ceil(L_b / 64) mapped
#     pages are pushed, sequences in batch order and blocks in ascending
#     order, and its block_table entries become -1.
# A call that cannot be satisfied changes nothing and reports why: status 1
# when the free pages do not suffice (reserve) or the stack would overflow
# (release: pages given back twice), status 2 when a table or length is out
# of range (a length past 64 * max_pages, a page id outside the pool).
# ----------------------------------------------------------------------------

def _pages(n_tokens: int) -> int:
    return (n_tokens + PAGE_SIZE - 1) // PAGE_SIZE if n_tokens > 0 else 0


def pages_init_ref(num_pages: int):
    """A pool with every page free.  Returns (free_pages int64 [num_pages],
    count)."""
    return np.arange(num_pages - 1, -1, -1, dtype=np.int64), num_pages


def pages_reserve_ref(free_pages, count: int, cache_seqlens, s_new: int, block_table):
    """Map the pages the next s_new tokens of every sequence need.  Returns
    (free_pages, count, block_table, status, pages handed out); on a status
    other than 0 the inputs come back unchanged."""
    fp = np.array(free_pages, dtype=np.int64, copy=True)
    bt = np.array(block_table, copy=True)
    L = np.asarray(cache_seqlens).astype(np.int64)
    B, max_pages = bt.shape
    needs = []
    for b in range(B):
        if L[b] < 0 or _pages(int(L[b]) + s_new) > max_pages:
            return np.array(free_pages, copy=True), count, np.array(block_table, copy=True), 2, 0
        needs.append((_pages(int(L[b])), _pages(int(L[b]) + s_new)))
    total = sum(want - have for have, want in needs)
    if total > count:
        return np.array(free_pages, copy=True), count, np.array(block_table, copy=True), 1, total
    top = count
    for b, (have, want) in enumerate(needs):
        for j in range(have, want):
            top -= 1
            bt[b, j] = fp[top]
    return fp, top, bt, 0, total


def pages_release_ref(free_pages, count: int, cache_seqlens, release, block_table, num_pages: int):
    """Give back the pages of every sequence whose release flag is set.
    Returns (free_pages, count, block_table, status, pages taken back)."""
    fp = np.array(free_pages, dtype=np.int64, copy=True)
    bt = np.array(block_table, copy=True)
    L = np.asarray(cache_seqlens).astype(np.int64)
    B, max_pages = bt.shape
    total = 0
    for b in range(B):
        if not release[b]:
            continue
        n = _pages(int(L[b]))
        if L[b] < 0 or n > max_pages or any(not 0 <= int(bt[b, j]) < num_pages for j in range(n)):
            return np.array(free_pages, copy=True), count, np.array(block_table, copy=True), 2, 0
        total += n
    if count + total > num_pages:
        return np.array(free_pages, copy=True), count, np.array(block_table, copy=True), 1, total
    top = count
    for b in range(B):
        if not release[b]:
            continue
        for j in range(_pages(int(L[b]))):
            fp[top] = bt[b, j]
            top += 1
            bt[b, j] = -1
    return fp, top, bt, 0, total


# ----------------------------------------------------------------------------
# fp8 cache: OCP E4M3 ("E4M3FN": 1 sign, 4 exponent bits with bias 7, 3
# mantissa bits; no infinities; 0x7F / 0xFF are NaN; largest finite 448;
# subnormals k * 2^-9).  The cache holds e4m3(clamp(x * inv_scale)) for one
# fp32 scale per cache, x * inv_scale computed in fp32 and clamped to
# [-448, 448] before rounding to nearest even, so every finite input maps to
# a finite code; an element's value is decode(code) * scale.
# ----------------------------------------------------------------------------

FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode_ref(codes) -> np.ndarray:
    """Value of each E4M3FN byte (NaN for 0x7F / 0xFF), from the format's
    definition: sign * 2^(e - 7) * (1 + m / 8) for e > 0, sign * 2^-6 * m / 8
    for e = 0."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e > 0, np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)), np.ldexp(m / 8.0, -6))
    val = sign * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


_E4M3_POS = fp8_e4m3_decode_ref(np.arange(0x7F))      # the 127 non-negative finite codes, ascending


def fp8_e4m3_encode_ref(x) -> np.ndarray:
    """Nearest E4M3FN code to each value (ties to the even code), after
    clamping to [-448, 448]; a NaN maps to the NaN code 0xFF."""
    v = np.asarray(x, dtype=np.float64)
    nan = np.isnan(v)
    a = np.clip(np.abs(np.where(nan, 0.0, v)), 0.0, FP8_E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0.0, 0, code)
    neg = np.signbit(v) & ~nan
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, 0xFF, code)                       # NaN in, NaN code out (0xFF)
    return code.astype(np.uint8)


def kvcache_append_fp8_ref(kvcache_fp8, block_table, cache_seqlens, kv_new, inv_scale):
    """:func:`kvcache_append_ref` into an fp8 cache: each new value x (bf16)
    becomes e4m3(clamp(float32(x) * float32(inv_scale))), the product in fp32.
    Returns (new cache codes, rows not written)."""
    new = np.asarray(as_f64(kv_new), dtype=np.float32)
    codes = fp8_e4m3_encode_ref((new * np.float32(inv_scale)).astype(np.float32))
    return kvcache_append_ref(kvcache_fp8, block_table, cache_seqlens, codes)


def mla_decode_fp8_ref(q, kvcache_fp8, kv_scale, block_table, cache_seqlens, dv: int = 512, causal: bool = False,
                       softmax_scale: float | None = None, batch_subset=None):
    """:func:`mla_decode_ref` over the fp8 cache's values, decode(code) *
    kv_scale, exactly as the cache defines them."""
    vals = fp8_e4m3_decode_ref(kvcache_fp8) * float(kv_scale)
    return mla_decode_ref(q, vals, block_table, cache_seqlens, dv, causal=causal, softmax_scale=softmax_scale,
                          batch_subset=batch_subset)
