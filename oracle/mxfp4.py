"""MXFP4: OCP microscaling FP4 (e2m1 elements, one E8M0 scale per block of
32), the block quantiser, and the exact block-scaled GEMM.

Test infrastructure only (see the package docstring).

The pages' mixed-precision band runs the norm-fed GEMMs in NVFP4 with
dynamic block scales and keeps the down projection in static FP8
(flashrt-structures 0.2.0, impls/adarms_stack/fp8_chain.py: the ``BANDS``
table, the ``fp4`` row, and ``_quantize``: block-scaled FP4 weights for
the norm-fed projections). NVFP4 is an NVIDIA format; the gfx950 matrix
cores take the OCP MX formats natively, so this band uses MXFP4, written
here from the OCP Microscaling Formats (MX) v1.0 specification:

- element e2m1: sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, bit 3 the sign; no inf/NaN;
- scale E8M0: the value 2^(s - 127) for byte s, 0xFF = NaN;
- a block of 32 consecutive values shares one scale;
- conversion (the specification's rule): shared exponent
  ``floor(log2(max|v|)) - 2`` (2 = the largest e2m1 exponent), clamped to
  the E8M0 range; each element is ``v / 2^shared`` rounded to nearest even
  on the e2m1 grid, saturating at +-6.

Readings where the pages and the specification leave a step open:
- blocks run along the GEMM's reduction axis: activation rows in 32-column
  blocks, weight rows (``[N, K]``) in 32-element blocks of K;
- the block maximum is taken of the fp32 values (the producer's y rounded
  to fp32, the weights decoded from bf16), so the scale is decided in fp32;
- a block whose maximum is 0 gets the smallest scale (byte 0) and zero
  codes; a NaN in a block makes its scale byte 0xFF;
- codes are stored two per byte, the lower-indexed element in the low
  nibble; scales one byte per block, stored run-major ``[K/256, rows, 8]``
  with each run of 8 blocks in the order 0, 2, 4, 6, 1, 3, 5, 7
  (``scales_to_gemm_order``: the library's layout, in which the GEMM reads
  a whole row block's scales for one K range as one contiguous piece);
- a NaN or an infinity in a block makes its scale byte 0xFF.
"""

from __future__ import annotations

import numpy as np

FP4_MAX = 6.0
BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """4-bit codes (0..15, any integer array) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v):
    """float -> e2m1 code, round to nearest with ties to the even code
    (even mantissa bit), saturating at +-6; the sign is kept (a negative
    value that rounds to zero gives -0, code 8); NaN is not representable
    and is rejected."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1 has no NaN")
    a = np.minimum(np.abs(v), FP4_MAX)
    # distance to every grid point; ties go to the even code index (the
    # grid's even indices are exactly the even-mantissa values)
    d = np.abs(a[..., None] - E2M1_VALUES)
    best = np.min(d, axis=-1, keepdims=True)
    cand = d == best
    idx = np.where(cand.sum(-1) > 1, np.argmax(cand & (np.arange(8) % 2 == 0), -1),
                   np.argmax(cand, -1))
    sign = np.signbit(v).astype(np.int64) << 3
    return (idx | sign).astype(np.uint8)


def e8m0_decode(s):
    s = np.asarray(s).astype(np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, (s - 127).astype(np.int32)))


def block_scale_exponent(amax):
    """OCP MX shared exponent for FP4: floor(log2(amax)) - 2, clamped to
    [-127, 127]; amax 0 -> -127. ``amax`` float32 (decided in fp32);
    floor(log2) is read exactly from the binary exponent (frexp)."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = m * 2^ex, m in [0.5, 1)
    e = np.where(a > 0, ex - 1, -1000)
    return np.clip(e - 2, -127, 127).astype(np.int64)


def quantize_mxfp4(v):
    """Block-quantise ``v`` (``[rows, K]``, K a multiple of 32) along its last
    axis. The values are taken in fp32. Returns ``(codes [rows, K] 0..15,
    scales [rows, K/32] E8M0 bytes)``."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    rows, K = v32.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = v32.reshape(rows, K // BLOCK, BLOCK)
    nan = (~np.isfinite(blocks)).any(-1)
    amax = np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0)), axis=-1)
    e = block_scale_exponent(amax)
    scales = np.where(nan, 255, e + 127).astype(np.uint8)
    # v / 2^e is exact (a power-of-two scaling of an fp32 value)
    q = blocks.astype(np.float64) / np.ldexp(1.0, e.astype(np.int32))[..., None]
    q = np.where(np.isfinite(q), q, 0.0)
    codes = e2m1_encode(q).reshape(rows, K)
    return codes, scales


def dequantize_mxfp4(codes, scales):
    c = np.asarray(codes)
    rows, K = c.shape
    vals = e2m1_decode(c).reshape(rows, K // BLOCK, BLOCK)
    return (vals * e8m0_decode(scales)[..., None]).reshape(rows, K)


def pack_nibbles(codes):
    """[rows, K] codes -> [rows, K/2] bytes (element 2j in the low nibble)."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


_RUN = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def scales_to_gemm_order(scales):
    """The library's scale layout: ``[K/256, rows, 8]`` (run-major: the 8
    block scales of each run of 256 elements of a row sit together, and the
    runs of all rows for one K range are contiguous), each run reordered to
    blocks 0, 2, 4, 6, 1, 3, 5, 7. ``scales`` is ``[rows, K/32]``."""
    s = np.asarray(scales)
    r, nb = s.shape
    return np.ascontiguousarray(s.reshape(r, nb // 8, 8)[:, :, _RUN].transpose(1, 0, 2))


def scales_from_gemm_order(stored):
    """Inverse of ``scales_to_gemm_order``: ``[K/256, rows, 8]`` -> ``[rows, K/32]``."""
    g = np.asarray(stored)
    runs, r, _ = g.shape
    out = np.empty((r, runs, 8), dtype=g.dtype)
    out[:, :, _RUN] = g.transpose(1, 0, 2)
    return out.reshape(r, runs * 8)


def gemm_mxfp4(a_codes, a_scales, b_codes, b_scales):
    """``acc[m, n] = sum_k dec(A[m,k]) * dec(B[n,k])`` over block-scaled
    MXFP4 operands (float64; exact whenever the blocks' scales keep the
    partial sums within 53 bits, as they do for any realistic data)."""
    A = dequantize_mxfp4(a_codes, a_scales)
    B = dequantize_mxfp4(b_codes, b_scales)
    return A @ B.T
