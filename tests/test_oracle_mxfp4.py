"""Pins for the oracle's MXFP4 codec, block quantiser and block-scaled GEMM
(CPU only), against the OCP MX v1.0 definitions written out independently
here: the e2m1 value formula from its bit fields, a per-element
nearest-value search with ties to the even code, the shared-exponent rule
checked by its defining inequality, the per-block error bound, and a
brute-force rational GEMM.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import mxfp4


def _e2m1_formula(code):
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))


def test_decode_matches_bit_field_formula():
    for c in range(16):
        assert mxfp4.e2m1_decode(np.array([c]))[0] == _e2m1_formula(c)
    assert mxfp4.e8m0_decode(np.array([127]))[0] == 1.0
    assert mxfp4.e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert mxfp4.e8m0_decode(np.array([254]))[0] == 2.0 ** 127
    assert np.isnan(mxfp4.e8m0_decode(np.array([255]))[0])


def _nearest_code(v):
    best = None
    for c in range(8):
        d = abs(min(abs(v), 6.0) - _e2m1_formula(c))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (8 if math.copysign(1.0, v) < 0 else 0)


def test_encode_is_nearest_with_ties_to_even():
    grid = sorted({_e2m1_formula(c) for c in range(8)})
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    vals = []
    for x in grid + mids + [0.1, 0.3, 6.5, 7.99, 100.0]:
        for eps in (0.0, 1e-9, -1e-9):
            vals += [x + eps, -(x + eps)]
    vals = [v for v in vals if v == v]
    got = mxfp4.e2m1_encode(np.array(vals))
    want = [_nearest_code(v) for v in vals]
    assert got.tolist() == want
    # the midpoints themselves: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0,
    # 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0
    assert mxfp4.e2m1_decode(mxfp4.e2m1_encode(np.array(mids))).tolist() == \
        [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    with pytest.raises(ValueError):
        mxfp4.e2m1_encode(np.array([np.nan]))


def test_shared_exponent_rule():
    rng = np.random.default_rng(1)
    a = np.abs(rng.standard_normal(10000) * 10.0 ** rng.uniform(-30, 30, 10000)).astype(np.float32)
    a = np.concatenate([a, np.float32([1.0, 2.0, 6.0, 8.0, 0.75, 2.0 ** -126, 2.0 ** -140])])
    e = mxfp4.block_scale_exponent(a)
    for ai, ei in zip(a.astype(np.float64), e):
        f = int(ei) + 2             # floor(log2(a)) unless clamped
        if -125 <= ei <= 127:
            assert 2.0 ** f <= ai < 2.0 ** (f + 1)
        else:
            assert ei in (-127, 127)
    assert mxfp4.block_scale_exponent(np.float32([0.0]))[0] == -127


def test_quantize_examples_and_error_bound():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((4, 128)) * np.array([1e-3, 1.0, 7.0, 1e4])[:, None]
    v[0, :32] = 0.0
    codes, scales = mxfp4.quantize_mxfp4(v)
    assert scales[0, 0] == 0 and (codes[0, :32] & 7 == 0).all()
    deq = mxfp4.dequantize_mxfp4(codes, scales)
    X = mxfp4.e8m0_decode(scales).repeat(32, axis=1)
    q = np.abs(v.astype(np.float32).astype(np.float64) / X)
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    ok = q <= 6.0
    assert np.all(np.abs(deq - v)[ok] <= 0.5 * step[ok] * X[ok] * (1 + 1e-12))
    # every non-zero block's largest element lands on 4 or 6 (amax / X in [4, 8))
    blocks = np.abs(codes.reshape(4, 4, 32) & 7)
    amax_code = blocks.max(-1)
    assert set(amax_code[1:].ravel().tolist()) <= {6, 7}
    # exact examples: a block holding 6 and 1 keeps both; 7.9 saturates to 6
    ex = np.zeros((1, 32))
    ex[0, :3] = [6.0, 1.0, 7.9]
    c, s = mxfp4.quantize_mxfp4(ex)
    assert s[0, 0] == 127 and mxfp4.e2m1_decode(c[0, :3]).tolist() == [6.0, 1.0, 6.0]


def test_nibble_order():
    c = np.array([[1, 2, 15, 8]], np.uint8)
    p = mxfp4.pack_nibbles(c)
    assert p.tolist() == [[0x21, 0x8F]]
    assert np.array_equal(mxfp4.unpack_nibbles(p), c)


def test_gemm_brute_force():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((2, 64)) * 3
    b = rng.standard_normal((3, 64)) * 0.1
    ac, as_ = mxfp4.quantize_mxfp4(a)
    bc, bs = mxfp4.quantize_mxfp4(b)
    got = mxfp4.gemm_mxfp4(ac, as_, bc, bs)
    for m in range(2):
        for n in range(3):
            acc = Fraction(0)
            for k in range(64):
                xa = Fraction(_e2m1_formula(int(ac[m, k]))) * Fraction(2) ** (int(as_[m, k // 32]) - 127)
                xb = Fraction(_e2m1_formula(int(bc[n, k]))) * Fraction(2) ** (int(bs[n, k // 32]) - 127)
                acc += xa * xb
            assert got[m, n] == float(acc)


def test_scale_order_round_trip():
    s = np.arange(2 * 16, dtype=np.uint8).reshape(2, 16)
    g = mxfp4.scales_to_gemm_order(s)
    assert g.shape == (2, 2, 8)
    assert g[0, 0].tolist() == [0, 2, 4, 6, 1, 3, 5, 7]       # run 0 of row 0
    assert g[0, 1].tolist() == [16, 18, 20, 22, 17, 19, 21, 23]  # run 0 of row 1
    assert g[1, 1].tolist() == [24, 26, 28, 30, 25, 27, 29, 31]
    assert np.array_equal(mxfp4.scales_from_gemm_order(g), s)


def test_non_finite_block_gets_nan_scale():
    v = np.zeros((1, 64))
    v[0, 3] = np.inf
    v[0, 40] = np.nan
    _, s = mxfp4.quantize_mxfp4(v)
    assert s.tolist() == [[255, 255]]
