"""bf16 and FP8 e4m3fn codecs, written from the formats' definitions.

Test infrastructure only (see the package docstring).

The pages use both formats without restating them: bf16 activations and
biases everywhere, and ``torch.float8_e4m3fn`` as the FP8 type of the packed
weights and the producer wire (flashrt-structures 0.2.0,
impls/qkv_pack/fp8_static.py ``_pack_weights``;
impls/modnorm_qkv_chain/fp8_ptok_table.py ``_q8`` and the FP8 maximum 448).
Neither page states a rounding mode; both casts are read as round to nearest,
ties to even, which is what torch's casts do.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0

# --------------------------------------------------------------------------
# bf16: the top 16 bits of an IEEE binary32.


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float32; exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Encode float32 to bf16 bits, round to nearest with ties to even.

    The kept part is the high half-word; the dropped low half-word ``lo``
    decides: above the halfway point 0x8000 round up, below it truncate, at
    it round up only if the kept part is odd. NaN stays a (quiet) NaN with
    its sign. Overflow past the largest finite bf16 becomes infinity, as
    round-to-nearest requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    hi = (u >> np.uint32(16)).astype(np.uint32)
    lo = u & np.uint32(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = (hi + up.astype(np.uint32)).astype(np.uint32)
    nan = np.isnan(x)
    out = np.where(nan, (hi & np.uint32(0x8000)) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


# --------------------------------------------------------------------------
# e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
# infinities; exponent 15 with mantissa 7 is NaN (codes 0x7F and 0xFF), so
# the largest finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).


def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
# non-negative finite magnitudes, indexed by code 0x00..0x7E (increasing)
_MAGS = E4M3_VALUES[:0x7F].copy()
# exact midpoints between neighbouring magnitudes (dyadic, exact in fp64)
_MIDS = (_MAGS[:-1] + _MAGS[1:]) / 2.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode e4m3fn codes to float64 (exact; NaN codes give NaN)."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Encode to e4m3fn: clamp to [-448, 448], then round to nearest with
    ties to the even code.

    The clamp is the pages' own step before the cast
    (``.clamp(-448, 448).to(float8_e4m3fn)`` in ``_pack_weights`` and
    ``_q8``). The magnitude is compared exactly against the midpoints between
    neighbouring codes; a value exactly on a midpoint takes the neighbour
    with the even code (even mantissa LSB). The sign is kept, so negative
    values that round to zero give -0 (0x80). NaN gives 0x7F / 0xFF by sign.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    nan = np.isnan(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)
    # i = number of midpoints strictly below a  -> candidate index
    lo = np.searchsorted(_MIDS, a, side="left")     # mids < a
    hi = np.searchsorted(_MIDS, a, side="right")    # mids <= a
    tie = hi > lo                                   # a is exactly a midpoint
    # on a tie the two neighbours are lo and lo+1: take the even one
    code = np.where(tie, np.where(lo % 2 == 0, lo, lo + 1), lo)
    code = code.astype(np.uint8)
    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, np.where(neg, 0xFF, 0x7F), code).astype(np.uint8)
    return code


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Signed ordinal of a code: +magnitude index, or minus it when the sign
    bit is set; +0 and -0 both map to 0. Neighbouring representable values
    differ by one ordinal, so |ordinal difference| counts e4m3 steps."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def e4m3_int(codes: np.ndarray) -> np.ndarray:
    """Integer ``k`` with value = k * 2^-9 (every finite e4m3 value is an
    integer multiple of the smallest subnormal 2^-9; |k| <= 229376)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 0x7
    k = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return np.where(c & 0x80, -k, k)
