"""Pins for the oracle's codecs (CPU only).

bf16 is pinned to torch's CPU cast (an independent library routine) on random
values and on every tie pattern; e4m3fn is pinned to the format's own code
points (tests/golden/e4m3fn_format.txt), to a brute-force nearest-code search
and to torch's CPU float8_e4m3fn cast.
"""

import os

import numpy as np
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_bf16_decode_all_patterns_roundtrip():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(codecs.f32_to_bf16(f[finite]), bits[finite])
    # decode places the pattern in the high half-word, exactly
    assert np.array_equal(f.view(np.uint32) >> 16, bits.astype(np.uint32))


def test_bf16_encode_matches_torch_random():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(codecs.f32_to_bf16(x), _torch_bf16(x))
    y = rng.standard_normal(200_000).astype(np.float32) * np.float32(37.0)
    assert np.array_equal(codecs.f32_to_bf16(y), _torch_bf16(y))


def test_bf16_encode_ties_to_even():
    rng = np.random.default_rng(6)
    hi = rng.integers(0, 0x7F7F, size=20000, dtype=np.uint32)
    for lo in (0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF):
        u = ((hi << 16) | lo).astype(np.uint32)
        for sign in (0, 0x80000000):
            x = (u | np.uint32(sign)).view(np.float32)
            x = x[np.isfinite(x)]
            assert np.array_equal(codecs.f32_to_bf16(x), _torch_bf16(x))
    # exact halfway cases by hand: 1 + 2^-8 is a tie between 1 and 1+2^-7
    assert codecs.f32_to_bf16(np.float32([1 + 2**-8]))[0] == 0x3F80
    assert codecs.f32_to_bf16(np.float32([1 + 3 * 2**-8]))[0] == 0x3F82


def test_bf16_encode_nan_and_overflow():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 3.4e38], np.float32)
    b = codecs.f32_to_bf16(x)
    assert np.isnan(codecs.bf16_to_f32(b[:2])).all()
    assert b[2] == 0x7F80 and b[3] == 0xFF80
    assert b[4] == 0x7F80   # rounds past the largest finite bf16


def test_e4m3_decode_matches_format_definition():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3fn_format.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    for c, v in rows:
        got = codecs.e4m3_decode(np.uint8([c]))[0]
        if np.isnan(v):
            assert np.isnan(got)
        else:
            assert got == v and np.signbit(got) == np.signbit(v), hex(c)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = codecs.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_int_is_value_in_units_of_2m9():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    k = codecs.e4m3_int(codes)
    assert np.array_equal(k * 2.0 ** -9, codecs.e4m3_decode(codes))
    assert np.abs(k).max() == 229376


def _brute_force_encode(v):
    """Nearest finite code by exhaustive search; ties to the even code."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = codecs.E4M3_VALUES[finite]
    out = np.empty(len(v), np.uint8)
    for i, x in enumerate(v):
        x = min(max(float(x), -448.0), 448.0)
        d = np.abs(vals - x)
        best = np.flatnonzero(d == d.min())
        cand = finite[best]
        # candidates at equal distance: +0/-0 pair (x == 0) or a tie
        if len(cand) > 1:
            if x == 0.0 or d.min() == 0.0:
                cand = cand[np.signbit(codecs.E4M3_VALUES[cand]) == np.signbit(x)]
            else:
                cand = cand[(cand & 1) == 0]
        c = int(cand[0])
        # a negative value that rounds to zero keeps its sign
        if (c & 0x7F) == 0 and np.signbit(x):
            c = 0x80
        out[i] = c
    return out


def _midpoint_set():
    mags = codecs.E4M3_VALUES[:0x7F]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)
    around = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                             np.nextafter(mids, np.float32(1e9)),
                             mags.astype(np.float32)])
    return np.concatenate([around, -around])


def test_e4m3_encode_brute_force_midpoints():
    v = _midpoint_set()
    assert np.array_equal(codecs.e4m3_encode(v), _brute_force_encode(v))


def test_e4m3_encode_brute_force_random():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(6000) * np.exp(rng.uniform(-12, 7, 6000)))
    v = v.astype(np.float32)
    v = np.concatenate([v, np.float32([500.0, -1e6, 448.0, 464.0, 463.99,
                                       2**-10, 2**-11, -2**-10, 0.0])])
    assert np.array_equal(codecs.e4m3_encode(v), _brute_force_encode(v))


def test_e4m3_encode_matches_torch_clamped_cast():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(1_000_000) *
         np.exp(rng.uniform(-14, 8, 1_000_000))).astype(np.float32)
    v = np.concatenate([v, _midpoint_set()])
    clamped = np.clip(v, -448, 448)
    assert np.array_equal(codecs.e4m3_encode(v), _torch_e4m3(clamped))


def test_e4m3_encode_specials():
    enc = codecs.e4m3_encode
    assert enc(np.float32([464.0]))[0] == 0x7E        # clamps, no NaN
    assert enc(np.float32([1e30]))[0] == 0x7E
    assert enc(np.float32([-1e30]))[0] == 0xFE
    assert enc(np.float32([1.0625]))[0] == 0x38       # tie -> even (1.0)
    assert enc(np.float32([1.1875]))[0] == 0x3A       # tie -> even (1.25)
    assert enc(np.float32([2**-10]))[0] == 0x00       # tie -> 0
    assert enc(np.float32([1.5 * 2**-9]))[0] == 0x02  # tie -> 2*2^-9
    assert enc(np.float32([-0.0]))[0] == 0x80
    assert enc(np.float32([np.nan]))[0] == 0x7F


def test_e4m3_ordinal_steps():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    o = codecs.e4m3_ordinal(codes)
    assert np.array_equal(np.diff(o), np.ones(0x7E, np.int64))
    assert codecs.e4m3_ordinal(np.uint8([0x80]))[0] == 0
    assert codecs.e4m3_ordinal(np.uint8([0x81]))[0] == -1
    # ordinal order equals value order over all finite codes
    fin = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    val = codecs.e4m3_decode(fin)
    ordv = codecs.e4m3_ordinal(fin)
    for a in range(len(fin)):
        assert ((ordv > ordv[a]) == (val > val[a])).all()
