"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a brute force of
the un-absorbed equations, a closed form, an invariant, or a library routine
(torch's scaled_dot_product_attention / logsumexp in float64).  The last block
plants plausible mistakes in the oracle (on the CPU) and shows that at least
one pin catches each of them.

Passages: deepseek.csdn.net FlashMLA article, section 2.2 -- equations (1)-(5)
(keys and values from the cached latent), (6)-(9) (query), the output
equation, and the matrix-absorption paragraph after it; section 4.2(1) (paged
cache with block_table, split-KV + combine kernels).
"""
import math

import numpy as np
import pytest
import torch

import oracle.mla_oracle as mo
from oracle.mla_oracle import (DEFAULT_SCALE, PAGE_SIZE, attend_range, lse_combine_ref,
                               mla_decode_ref)

D_C, D_H, D_HR = 512, 128, 64
D_QK = D_C + D_HR
D_MODEL = 24          # output width of W^O in the brute-force cases (any width works)


def _paged(rows_per_seq, rng, h_kv=1, extra_pages=2):
    """Pack per-sequence latent rows [L][h_kv][576] into a shuffled page pool."""
    n_pages = [(len(r) + PAGE_SIZE - 1) // PAGE_SIZE for r in rows_per_seq]
    pool = sum(n_pages) + extra_pages
    perm = rng.permutation(pool)
    kv = rng.standard_normal((pool, PAGE_SIZE, h_kv, D_QK)) * 1e3   # garbage in unused slots
    bt = np.full((len(rows_per_seq), max(max(n_pages), 1)), -1, dtype=np.int64)
    off = 0
    for b, rows in enumerate(rows_per_seq):
        for blk in range(n_pages[b]):
            page = perm[off]
            off += 1
            bt[b, blk] = page
            chunk = rows[blk * PAGE_SIZE:(blk + 1) * PAGE_SIZE]
            kv[page, :len(chunk)] = chunk
    return kv, bt


# ----------------------------------------------------------------------------
# P-1: brute-force un-absorbed MHA (equations (1)-(5), (9) and the output
# equation) equals the absorbed paged oracle after applying W^UV.
# ----------------------------------------------------------------------------

def _brute_force_case(seqlens, s_q, h_q, h_kv, causal, seed):
    rng = np.random.default_rng(seed)
    B, G = len(seqlens), h_q // h_kv
    c = [rng.standard_normal((L, h_kv, D_C)) for L in seqlens]           # c^KV_j per latent head
    kr = [rng.standard_normal((L, h_kv, D_HR)) for L in seqlens]         # k^R_j (RoPE already applied)
    w_uk = rng.standard_normal((h_q, D_H, D_C)) / math.sqrt(D_C)
    w_uv = rng.standard_normal((h_q, D_H, D_C)) / math.sqrt(D_C)
    qc = rng.standard_normal((B, s_q, h_q, D_H))
    qr = rng.standard_normal((B, s_q, h_q, D_HR))
    w_o = rng.standard_normal((D_MODEL, h_q * D_H)) / math.sqrt(h_q * D_H)

    # Un-absorbed: per head i, k_{j,i} = [W^UK_i c_j ; k^R_j], v_{j,i} = W^UV_i c_j,
    # q_{t,i} = [q^C ; q^R], o = sum_{j<=t} softmax(q.k / sqrt(d_h + d_h^R)) v.
    o_ref = np.zeros((B, s_q, h_q, D_H))
    lse_ref = np.full((B, h_q, s_q), -np.inf)
    for b, L in enumerate(seqlens):
        for t in range(s_q):
            pos = L - s_q + t                 # position of query token t in the sequence
            n_vis = min(L, pos + 1) if causal else L
            n_vis = max(n_vis, 0)
            for i in range(h_q):
                g = i // G
                if n_vis == 0:
                    continue
                scores = []
                vals = []
                for j in range(n_vis):
                    k = np.concatenate([w_uk[i] @ c[b][j, g], kr[b][j, g]])
                    q = np.concatenate([qc[b, t, i], qr[b, t, i]])
                    scores.append(float(q @ k) / math.sqrt(D_H + D_HR))
                    vals.append(w_uv[i] @ c[b][j, g])
                m = max(scores)
                z = math.fsum(math.exp(s - m) for s in scores)
                lse_ref[b, i, t] = m + math.log(z)
                o_ref[b, t, i] = sum(math.exp(s - m) / z * v for s, v in zip(scores, vals))
    # Second output equation, head by head: W^O [o_1; ...; o_n] is the sum over
    # heads i of W^O's column block i (columns i*d_h .. i*d_h + d_h - 1) times o_i.
    u_ref = np.zeros((B, s_q, D_MODEL))
    for b in range(B):
        for t in range(s_q):
            for i in range(h_q):
                u_ref[b, t] += w_o[:, i * D_H:(i + 1) * D_H] @ o_ref[b, t, i]

    # Absorbed: q~ = [W^UK^T q^C ; q^R], cached rows [c^KV ; k^R] in pages.
    T = B * s_q
    q_abs = mo.absorb_q_ref(qc.reshape(T, h_q, D_H), qr.reshape(T, h_q, D_HR),
                            np.ascontiguousarray(w_uk.transpose(0, 2, 1))).reshape(B, s_q, h_q, D_QK)
    rows = [np.concatenate([c[b], kr[b]], axis=-1) for b in range(B)]
    kv, bt = _paged(rows, rng, h_kv)
    O, LSE = mla_decode_ref(q_abs, kv, bt, np.asarray(seqlens), dv=D_C, causal=causal)
    o_from_latent = mo.absorb_o_ref(O.reshape(T, h_q, D_C), w_uv).reshape(B, s_q, h_q, D_H)
    u_abs = mo.out_proj_ref(o_from_latent.reshape(T, h_q, D_H), w_o).reshape(B, s_q, D_MODEL)
    return o_ref, lse_ref, o_from_latent, LSE, u_ref, u_abs


def _p1_error(seqlens, s_q, h_q, h_kv, causal, seed):
    o_ref, lse_ref, o_abs, lse_abs, u_ref, u_abs = _brute_force_case(seqlens, s_q, h_q, h_kv, causal, seed)
    scale = max(1.0, np.abs(o_ref).max())
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lse_abs) == fin).all()
    return max(np.abs(o_abs - o_ref).max() / scale, np.abs(lse_abs[fin] - lse_ref[fin]).max(),
               np.abs(u_abs - u_ref).max() / max(1.0, np.abs(u_ref).max()))


@pytest.mark.parametrize("seqlens,s_q,h_kv,causal", [
    ((5, 130), 1, 1, False),
    ((1, 65), 2, 1, True),
    ((64, 5), 2, 2, False),
    ((130, 64), 2, 1, True),
    ((1, 1), 2, 2, True),       # causal row 0 of a one-token cache sees nothing
    ((130, 200), 2, 1, True),
])
def test_p1_unabsorbed_brute_force(seqlens, s_q, h_kv, causal):
    assert _p1_error(seqlens, s_q, 4, h_kv, causal, seed=11) <= 1e-10


# ----------------------------------------------------------------------------
# P-2: softmax weights sum to one; LSE identity against an independent sum.
# ----------------------------------------------------------------------------

def test_p2_weights_sum_to_one_and_lse_identity():
    rng = np.random.default_rng(3)
    L, h_q = 7, 3
    rows = rng.standard_normal((L, 1, D_QK))
    q = rng.standard_normal((1, 1, h_q, D_QK))
    kv, bt = _paged([rows], rng)
    O, LSE, P = mla_decode_ref(q, kv, bt, np.array([L]), dv=512, return_p=True)
    for h in range(h_q):
        p = P[(0, 0, h)]
        assert abs(p.sum() - 1.0) <= 1e-12
        s = [DEFAULT_SCALE * math.fsum(q[0, 0, h, d] * rows[j, 0, d] for d in range(D_QK)) for j in range(L)]
        lse = math.log(math.fsum(math.exp(x) for x in s))
        assert abs(LSE[0, h, 0] - lse) <= 1e-12
        o = [math.fsum(math.exp(s[j] - lse) * rows[j, 0, d] for j in range(L)) for d in range(512)]
        np.testing.assert_allclose(O[0, 0, h], o, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P-3 constant latent, P-4 single token: closed forms.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("L", [1, 37, 64, 130])
def test_p3_constant_latent(L):
    rng = np.random.default_rng(L)
    u = rng.standard_normal(D_QK)
    q = rng.standard_normal((1, 2, 4, D_QK))
    kv, bt = _paged([np.tile(u, (L, 1, 1))], rng)
    O, LSE = mla_decode_ref(q, kv, bt, np.array([L]), dv=512)
    np.testing.assert_allclose(O, np.broadcast_to(u[:512], O.shape), rtol=0, atol=1e-12)
    expect = DEFAULT_SCALE * np.einsum("bthd,d->bht", q, u) + math.log(L)
    np.testing.assert_allclose(LSE, expect, rtol=0, atol=1e-12)


def test_p4_single_token():
    rng = np.random.default_rng(4)
    row = rng.standard_normal(D_QK)
    q = rng.standard_normal((1, 1, 8, D_QK))
    kv, bt = _paged([row[None, None, :]], rng)
    O, LSE = mla_decode_ref(q, kv, bt, np.array([1]), dv=512)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(row[:512], (8, 512)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE[0, :, 0], DEFAULT_SCALE * q[0, 0] @ row, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P-5: page-permutation invariance (bitwise).
# ----------------------------------------------------------------------------

def test_p5_page_permutation_bitwise():
    rng = np.random.default_rng(5)
    lens = [37, 130, 64]
    rows = [rng.standard_normal((L, 1, D_QK)) for L in lens]
    q = rng.standard_normal((3, 1, 8, D_QK))
    kv, bt = _paged(rows, rng)
    O1, L1 = mla_decode_ref(q, kv, bt, np.array(lens))
    perm = rng.permutation(kv.shape[0])
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    O2, L2 = mla_decode_ref(q, kv2, bt2, np.array(lens))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


# ----------------------------------------------------------------------------
# P-6: reduction to torch's scaled_dot_product_attention (float64, CPU).
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_p6_sdpa_reduction(causal):
    rng = np.random.default_rng(6)
    lens, s_q, h_q = [37, 130], 2, 4
    rows = [rng.standard_normal((L, 1, D_QK)) for L in lens]
    q = rng.standard_normal((2, s_q, h_q, D_QK))
    kv, bt = _paged(rows, rng)
    O, LSE = mla_decode_ref(q, kv, bt, np.array(lens), causal=causal)
    for b, L in enumerate(lens):
        K = torch.from_numpy(rows[b][:, 0, :])                     # [L, 576], logical order
        V = K[:, :512]
        Q = torch.from_numpy(q[b]).permute(1, 0, 2)                 # [h, s_q, 576]
        mask = torch.ones(s_q, L, dtype=torch.bool)
        if causal:
            mask = torch.arange(L)[None, :] <= (L - s_q + torch.arange(s_q))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K.expand(h_q, L, D_QK), V.expand(h_q, L, 512), attn_mask=mask, scale=DEFAULT_SCALE)
        s = (Q @ K.T) * DEFAULT_SCALE
        lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)   # [h, s_q]
        np.testing.assert_allclose(O[b], o.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[b], lse.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P-7: causal reductions.
# ----------------------------------------------------------------------------

def test_p7_causal_reductions():
    rng = np.random.default_rng(7)
    lens = [65, 3]
    rows = [rng.standard_normal((L, 1, D_QK)) for L in lens]
    kv, bt = _paged(rows, rng)
    q1 = rng.standard_normal((2, 1, 4, D_QK))
    a = mla_decode_ref(q1, kv, bt, np.array(lens), causal=True)
    b_ = mla_decode_ref(q1, kv, bt, np.array(lens), causal=False)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1])
    s_q = 3
    q3 = rng.standard_normal((2, s_q, 4, D_QK))
    O, LSE = mla_decode_ref(q3, kv, bt, np.array(lens), causal=True)
    for i in range(s_q):
        shorter = [L - s_q + i + 1 for L in lens]
        Oi, Li = mla_decode_ref(q3[:, i:i + 1], kv, bt, np.array(shorter), causal=False)
        # same math, but BLAS may block a longer score product differently
        np.testing.assert_allclose(O[:, i], Oi[:, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[:, :, i], Li[:, :, 0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# P-8: any partition of the keys, merged by the LSE formula, equals the whole.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("L,cuts", [(130, [64]), (300, [1, 64, 65, 200]), (9, [3, 4, 5, 8])])
def test_p8_split_combine_invariance(L, cuts):
    rng = np.random.default_rng(L)
    keys = rng.standard_normal((L, D_QK))
    rows = rng.standard_normal((6, D_QK))
    n_vis = [L, L, L - 1, L - 1, 1, L]          # includes rows that see few keys
    whole = attend_range(rows, keys, 0, L, n_vis, 512, DEFAULT_SCALE)
    bounds = [0] + cuts + [L]
    parts = [attend_range(rows, keys, lo, hi, n_vis, 512, DEFAULT_SCALE) for lo, hi in zip(bounds, bounds[1:])]
    O, lse = lse_combine_ref(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(O, whole[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, whole[1], rtol=0, atol=1e-12)


def test_p8_combine_of_empty_splits():
    O, lse = lse_combine_ref(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert (O == 0).all() and np.isneginf(lse).all()


# ----------------------------------------------------------------------------
# P-9: h_kv latent heads behave as h_kv independent single-head problems.
# ----------------------------------------------------------------------------

def test_p9_grouping():
    rng = np.random.default_rng(9)
    lens, h_kv, h_q = [70, 5], 2, 6
    rows = [rng.standard_normal((L, h_kv, D_QK)) for L in lens]
    q = rng.standard_normal((2, 2, h_q, D_QK))
    kv, bt = _paged(rows, rng, h_kv=h_kv)
    O, LSE = mla_decode_ref(q, kv, bt, np.array(lens), causal=True)
    G = h_q // h_kv
    for g in range(h_kv):
        Og, Lg = mla_decode_ref(q[:, :, g * G:(g + 1) * G], kv[:, :, g:g + 1], bt, np.array(lens), causal=True)
        np.testing.assert_array_equal(O[:, :, g * G:(g + 1) * G], Og)
        np.testing.assert_array_equal(LSE[:, g * G:(g + 1) * G], Lg)


# ----------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ----------------------------------------------------------------------------

def _pins_pass() -> bool:
    try:
        assert _p1_error((5, 130), 2, 4, 1, True, seed=2) <= 1e-10
        assert _p1_error((130, 200), 2, 2, 1, True, seed=12) <= 1e-10
        test_p3_constant_latent(37)
        test_p4_single_token()
        test_p6_sdpa_reduction(True)
    except AssertionError:
        return False
    return True


def _mutant_attend(kind):
    real = mo.attend

    def attend(q_rows, keys, n_vis, dv, scale, return_p=False):
        if kind == "drop_rope":
            q_rows = q_rows.copy()
            q_rows[:, 512:] = 0
        if kind == "v_from_wrong_columns":
            keys = np.concatenate([keys[:, 64:], keys[:, :64]], axis=1)
        res = real(q_rows, keys, n_vis, dv, scale, return_p)
        if kind == "lse_log2":
            res = (res[0], res[1] / math.log(2)) + tuple(res[2:])
        return res
    return attend


@pytest.mark.parametrize("kind", ["scale_576", "drop_rope", "v_from_wrong_columns", "lse_log2",
                                  "causal_off_by_one", "gather_ignores_block_table", "sign_flip_q"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    assert _pins_pass()
    if kind == "scale_576":
        monkeypatch.setattr(mo, "DEFAULT_SCALE", 1 / math.sqrt(576))
    elif kind == "causal_off_by_one":
        real = mo.visible_keys
        monkeypatch.setattr(mo, "visible_keys", lambda L, s_q, i, c: max(0, real(L, s_q, i, c) - (1 if c else 0)))
    elif kind == "gather_ignores_block_table":
        real_g = mo.gather_latent_rows
        monkeypatch.setattr(mo, "gather_latent_rows",
                            lambda kv, row, L, g: real_g(kv, np.sort(np.where(np.asarray(row) >= 0, row, 1 << 30)), L, g))
    elif kind == "sign_flip_q":
        real_a = mo.attend
        monkeypatch.setattr(mo, "attend", lambda q, k, n, dv, s, rp=False: real_a(-q, k, n, dv, s, rp))
    else:
        monkeypatch.setattr(mo, "attend", _mutant_attend(kind))
    assert not _pins_pass(), f"planted mistake {kind!r} slipped through every pin"


@pytest.mark.parametrize("kind", ["rope_dropped", "weight_untransposed_head", "output_heads_rolled"])
def test_planted_absorption_mistakes_are_caught(kind, monkeypatch):
    """P-1 runs its absorbed side through absorb_q_ref and absorb_o_ref, so it
    pins them against the un-absorbed equations: plausible mistakes in them
    fail it."""
    aq, ao = mo.absorb_q_ref, mo.absorb_o_ref
    if kind == "rope_dropped":
        monkeypatch.setattr(mo, "absorb_q_ref", lambda qn, qr, w: aq(qn, 0 * np.asarray(qr), w))
    elif kind == "weight_untransposed_head":
        monkeypatch.setattr(mo, "absorb_q_ref", lambda qn, qr, w: aq(qn, qr, np.roll(w, 1, axis=0)))
    else:
        monkeypatch.setattr(mo, "absorb_o_ref", lambda o, w: np.roll(ao(o, w), 1, axis=1))
    assert _p1_error((5, 70), 1, 4, 1, False, seed=3) > 1e-3


@pytest.mark.parametrize("kind", ["heads_reversed", "head_dims_interleaved", "weight_blocks_rolled"])
def test_planted_output_projection_mistakes_are_caught(kind, monkeypatch):
    """P-1 also runs the absorbed side through out_proj_ref and compares it
    with W^O applied head block by head block to the un-absorbed outputs, so
    a wrong stacking order of the heads, or of W^O's column blocks, fails."""
    op = mo.out_proj_ref
    if kind == "heads_reversed":
        monkeypatch.setattr(mo, "out_proj_ref", lambda o, w: op(np.asarray(o)[:, ::-1, :], w))
    elif kind == "head_dims_interleaved":
        monkeypatch.setattr(mo, "out_proj_ref",
                            lambda o, w: op(np.ascontiguousarray(np.asarray(o).transpose(0, 2, 1)).reshape(np.shape(o)), w))
    else:
        monkeypatch.setattr(mo, "out_proj_ref", lambda o, w: op(o, np.roll(np.asarray(w), D_H, axis=1)))
    assert _p1_error((5, 70), 1, 4, 1, False, seed=3) > 1e-3
