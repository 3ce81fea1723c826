"""Pins of the oracle's fp8 cache functions against the OCP E4M3 format's
definition (8 bits: sign, 4 exponent bits with bias 7, 3 mantissa bits; no
infinities; S.1111.111 is NaN; largest finite 448): specific code values, the
format's structure (symmetry, monotonicity, spacing), round trips, round to
nearest even at midpoints, clamping, and the fp8 decode's reduction to the
bf16 decode on the dequantized values.  Planted mistakes must fail them."""
import math

import numpy as np
import pytest

import oracle.mla_oracle as mo


def test_decode_known_codes():
    d = mo.fp8_e4m3_decode_ref
    expect = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
              0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x78: 256.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in expect.items():
        assert d(c) == v, hex(c)
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert math.copysign(1.0, d(0x80)) == -1.0 and d(0x80) == 0.0


def test_decode_structure():
    vals = mo.fp8_e4m3_decode_ref(np.arange(0x7F))
    assert (np.diff(vals) > 0).all()                                   # monotone over 0x00..0x7E
    assert (mo.fp8_e4m3_decode_ref(np.arange(0x7F) | 0x80) == -vals).all()   # sign bit
    # spacing: 2^(e-10) within binade e (e = 1..15), 2^-9 among subnormals
    for c in range(0x01, 0x7E):
        e = max((c >> 3) & 0xF, 1)
        assert vals[c + 1] - vals[c] == 2.0 ** (e - 10) or (c & 7) == 7, hex(c)


def test_encode_round_trip_and_nearest():
    enc, dec = mo.fp8_e4m3_encode_ref, mo.fp8_e4m3_decode_ref
    codes = np.concatenate([np.arange(0x7F), np.arange(0x7F) | 0x80])
    codes = codes[codes != 0x80]                                        # -0 encodes as 0x80, checked below
    assert (enc(dec(codes)) == codes).all()
    assert enc(-0.0) == 0x80
    rng = np.random.default_rng(0)
    x = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-12, 1, 20000))
    got = dec(enc(x))
    # no code lies strictly closer to x than the chosen one
    allv = dec(np.arange(0x7F))
    allv = np.concatenate([-allv[::-1], allv])
    best = np.abs(allv[None, :] - x[:, None]).min(axis=1)
    assert np.allclose(np.abs(got - x), best, rtol=0, atol=0)


def test_encode_ties_to_even_and_clamps():
    enc = mo.fp8_e4m3_encode_ref
    assert enc(1.0625) == 0x38                 # midway 1.0 (even) / 1.125
    assert enc(1.1875) == 0x3A                 # midway 1.125 / 1.25 (even)
    assert enc(2.0 ** -10) == 0x00             # midway 0 / 2^-9
    assert enc(3 * 2.0 ** -10) == 0x02         # midway 2^-9 / 2^-8 (even)
    assert enc(272.0) == 0x78                  # midway 256 (even) / 288
    assert enc(464.0) == 0x7E and enc(480.0) == 0x7E and enc(1e30) == 0x7E and enc(np.inf) == 0x7E
    assert enc(-1e30) == 0xFE and enc(-np.inf) == 0xFE
    assert enc(np.nan) == 0xFF


def test_append_fp8_worked_example():
    """One row appended at position 3 of a one-page cache, scale 0.5
    (inv_scale 2): 1.5 -> 3.0 = 0x44; -0.125 -> -0.25 = 0xA8; 300 -> 600,
    clamped to 448 = 0x7E; 2^-11 -> 2^-10, midway 0 and 2^-9 -> 0x00."""
    cache = np.zeros((1, 64, 1, 4), dtype=np.uint8)
    row = np.array([[[[1.5, -0.125, 300.0, 2.0 ** -11]]]])
    out, bad = mo.kvcache_append_fp8_ref(cache, np.array([[0]]), np.array([3]), row, 2.0)
    assert bad == 0
    assert out[0, 3, 0].tolist() == [0x44, 0xA8, 0x7E, 0x00]
    assert (np.delete(out[0], 3, axis=0) == 0).all()


def test_fp8_decode_constant_latent_and_scale():
    """All cached rows the same code vector u (exactly representable):
    O = decode(u)[:512] * scale for every query, and LSE = sigma * scale *
    q.decode(u) + ln L (the constant-latent closed form on the fp8 values)."""
    rng = np.random.default_rng(2)
    L, h = 70, 4
    u = rng.integers(0, 0x7E, 576).astype(np.uint8) | (rng.integers(0, 2, 576).astype(np.uint8) << 7)
    cache = np.broadcast_to(u, (2, 64, 1, 576)).copy()
    q = rng.standard_normal((1, 1, h, 576))
    scale = 0.75
    O, LSE = mo.mla_decode_fp8_ref(q, cache, scale, np.array([[1, 0]]), np.array([L]))
    vu = mo.fp8_e4m3_decode_ref(u) * scale
    assert np.allclose(O[0, 0], np.broadcast_to(vu[:512], (h, 512)), rtol=0, atol=1e-12)
    sig = 1 / math.sqrt(192)
    assert np.allclose(LSE[0, :, 0], sig * (q[0, 0] @ vu) + math.log(L), rtol=0, atol=1e-10)


@pytest.mark.parametrize("kind", ["bias_8", "no_tie_even", "no_clamp", "mantissa_4"])
def test_planted_fp8_mistakes_are_caught(kind, monkeypatch):
    real_dec, real_enc = mo.fp8_e4m3_decode_ref, mo.fp8_e4m3_encode_ref
    if kind == "bias_8":
        monkeypatch.setattr(mo, "fp8_e4m3_decode_ref", lambda c: real_dec(c) / 2)
    elif kind == "mantissa_4":
        monkeypatch.setattr(mo, "fp8_e4m3_decode_ref",
                            lambda c: np.where(np.asarray(c) & 1, real_dec(np.asarray(c) & ~1), real_dec(c)))
    elif kind == "no_tie_even":
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            return real_enc(np.nextafter(x, np.where(x >= 0, np.inf, -np.inf)))     # ties away from zero
        monkeypatch.setattr(mo, "fp8_e4m3_encode_ref", enc)
    else:
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            return np.where(np.abs(x) > 464, 0x7F, real_enc(x)).astype(np.uint8)
        monkeypatch.setattr(mo, "fp8_e4m3_encode_ref", enc)
    failed = 0
    for t in (test_decode_known_codes, test_decode_structure, test_encode_round_trip_and_nearest,
              test_encode_ties_to_even_and_clamps, test_append_fp8_worked_example):
        try:
            t()
        except AssertionError:
            failed += 1
    assert failed, f"planted mistake {kind!r} slipped through"
