"""Pins for the uint4 group-quantization oracle.

Independent checks: exact rational arithmetic (fractions.Fraction) with a
brute-force search over every fp16 value for the scale and over all 16 codes
for each element, the exact round-trip bound |x - x_hat| <= s16/2, closed-form
groups (0..15 gives scale 1 and the identity; half steps round to even), the
nibble order, degenerate groups, and integer data that survives quantization
unchanged (then kv4 attention equals dense attention on the originals).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import decode_attention, dequantize_kv4, kv4_attention, quantize_kv4
from oracle.kv4 import unpack_codes

# every finite binary16 value, as exact rationals, sorted by value
_ALL16 = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
_FIN16 = sorted({Fraction(float(x)) for x in _ALL16 if np.isfinite(x)})


def _nearest_fp16(x: Fraction) -> Fraction:
    import bisect
    i = bisect.bisect_left(_FIN16, x)
    cands = [c for c in _FIN16[max(0, i - 1):i + 2]]
    best = min(abs(c - x) for c in cands)
    ties = [c for c in cands if abs(c - x) == best]
    if len(ties) == 1:
        return ties[0]
    # tie: the one whose fp16 bit pattern is even
    ev = [c for c in ties
          if int(np.float16(float(c)).view(np.uint16)) % 2 == 0]
    return ev[0]


def _brute_group(xs):
    fx = [Fraction(float(x)) for x in xs]
    mn, mx = min(fx), max(fx)
    s = _nearest_fp16((mx - mn) / 15)
    codes = []
    for x in fx:
        if s == 0:
            codes.append(0)
            continue
        errs = [abs(x - (mn + c * s)) for c in range(16)]
        best = min(errs)
        cs = [c for c in range(16) if errs[c] == best]
        codes.append(cs[0] if len(cs) == 1 else [c for c in cs if c % 2 == 0][0])
    return mn, s, codes


def _groups_under_test():
    rng = np.random.default_rng(11)
    gs = [rng.standard_normal(64).astype(np.float16) for _ in range(6)]
    gs.append((rng.standard_normal(64) * 1e-5).astype(np.float16))   # subnormal-ish
    gs.append((rng.standard_normal(64) * 300).astype(np.float16))
    # deliberate ties: values on half steps of an integer grid
    t = np.concatenate([np.arange(16), np.arange(16) + 0.5, np.arange(16) * 0.25,
                        np.arange(16) * 0.75]).astype(np.float16)
    gs.append(t)
    return gs


def test_quantize_matches_exact_rational_brute_force():
    for g in _groups_under_test():
        codes, gmin, gscale = quantize_kv4(g[None, :])
        mn, s, want = _brute_group(g)
        assert Fraction(float(gmin[0, 0])) == mn
        assert Fraction(float(gscale[0, 0])) == s
        got = unpack_codes(codes)[0]
        assert list(int(c) for c in got) == want


def test_round_trip_error_at_most_half_a_step():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((50, 128)).astype(np.float16)
    codes, gmin, gscale = quantize_kv4(x)
    c = unpack_codes(codes).reshape(50, 2, 64)
    for r in range(50):
        for g in range(2):
            mn = Fraction(float(gmin[r, g]))
            s = Fraction(float(gscale[r, g]))
            for i in range(64):
                xv = Fraction(float(x[r, g * 64 + i]))
                assert abs(xv - (mn + int(c[r, g, i]) * s)) <= s / 2


def test_identity_group_and_nibble_order():
    g = np.tile(np.arange(16, dtype=np.float16), 4)[None, :]
    codes, gmin, gscale = quantize_kv4(g)
    assert float(gmin[0, 0]) == 0.0 and float(gscale[0, 0]) == 1.0
    assert list(codes[0, :8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    np.testing.assert_array_equal(dequantize_kv4(codes, gmin, gscale), g)


def test_half_steps_round_to_even():
    g = np.zeros(64, dtype=np.float16)
    g[1] = 15.0
    g[2], g[3], g[4], g[5] = 2.5, 3.5, 0.5, 14.5
    codes, gmin, gscale = quantize_kv4(g[None, :])
    c = unpack_codes(codes)[0]
    assert float(gscale[0, 0]) == 1.0
    assert (int(c[2]), int(c[3]), int(c[4]), int(c[5])) == (2, 4, 0, 14)


def test_constant_group_has_zero_scale_and_zero_codes():
    g = np.full((1, 64), -1.25, dtype=np.float16)
    codes, gmin, gscale = quantize_kv4(g)
    assert float(gscale[0, 0]) == 0.0 and float(gmin[0, 0]) == -1.25
    assert not codes.any()
    np.testing.assert_array_equal(dequantize_kv4(codes, gmin, gscale), g)


def test_dequantize_rounds_once_to_fp16():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((4, 64)) * 3).astype(np.float16)
    codes, gmin, gscale = quantize_kv4(x)
    xh = dequantize_kv4(codes, gmin, gscale)
    c = unpack_codes(codes)
    for r in range(4):
        mn = Fraction(float(gmin[r, 0]))
        s = Fraction(float(gscale[r, 0]))
        for i in range(64):
            assert Fraction(float(xh[r, i])) == _nearest_fp16(mn + int(c[r, i]) * s)


def test_groups_run_along_the_hidden_dim_of_each_row():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((3, 128)).astype(np.float16)
    x[1, 64:] *= 100                                  # second group of row 1 only
    _, gmin, gscale = quantize_kv4(x)
    assert gscale.shape == (3, 2)
    assert float(gscale[1, 1]) > 10 * float(gscale[1, 0])
    assert float(gscale[0, 1]) < 10 * float(gscale[0, 0])


def test_kv4_attention_equals_dense_on_integer_data():
    rng = np.random.default_rng(15)
    B, H, N, D = 2, 2, 20, 128
    k = rng.integers(0, 16, size=(B, H, N, D)).astype(np.float16)
    v = rng.integers(-7, 9, size=(B, H, N, D)).astype(np.float16)
    k[..., 0] = 0
    k[..., 1] = 15                       # every key group spans exactly 0..15
    k[..., 64] = 0
    k[..., 65] = 15
    v[..., 0::64] = -7
    v[..., 1::64] = 8
    q = rng.standard_normal((B, H, D)).astype(np.float16).astype(np.float64)
    kc, kmn, ksc = quantize_kv4(k)
    vc, vmn, vsc = quantize_kv4(v)
    np.testing.assert_array_equal(dequantize_kv4(kc, kmn, ksc), k)
    np.testing.assert_array_equal(dequantize_kv4(vc, vmn, vsc), v)
    o = kv4_attention(q, kc, kmn, ksc, vc, vmn, vsc, 0.1)
    ref = decode_attention(q, k.astype(np.float64), v.astype(np.float64), 0.1)
    np.testing.assert_allclose(o, ref, atol=1e-14)


def test_rejects_rows_not_multiple_of_64():
    with pytest.raises(AssertionError):
        quantize_kv4(np.zeros((1, 96), dtype=np.float16))
