"""Packed FP8 GEMM: exact accumulation, dequant + bias epilogue, split.

Test infrastructure only (see the package docstring).

Follows the pages' packed-projection calls (flashrt-structures 0.2.0,
impls/qkv_pack/fp8_static.py ``PackedLinear._run``: ``fp8_gemm_bf16(x8, w8,
act_scale, w_scale)`` or ``fp8_linear_bias_bf16(x8, w8, bias_cat, act_scale,
w_scale)`` into the ``[M, sum N_i]`` output, later siblings read from column
offsets ``off_i = sum_{t<i} N_t``; impls/adarms_stack/fp8_chain.py folds the
two scales into ``alpha = act_scale * w_scale``):

    out[m, n] = alpha * sum_k dec(x8[m, k]) * dec(W8[n, k]) + bias[n]

Every e4m3 value is an integer multiple of 2^-9 with |k| <= 229376 < 2^18,
so each product is an integer multiple of 2^-18 below 2^36 in magnitude and
a K-term sum stays below 2^53 for K <= 2^17: the fp64 matmul of the integer
code values is therefore exact, whatever its summation order. The GEMM is
the plain definition; there is no other rounding until the epilogue.

Reading where the pages are silent: the fused bias entry rounds once, so the
reference output is ``alpha * acc + bias`` formed in float64 (relative error
at most 2^-52, far below either output format's rounding) and rounded once
to the output type (bf16 by round-to-nearest-even); ``alpha`` is
``fl32(act_scale * w_scale)``.
"""

from __future__ import annotations

import numpy as np

from .codecs import e4m3_int, bf16_to_f32, f32_to_bf16

_TWO_M18 = 2.0 ** -18
_COLS_PER_BLOCK = 2048


def gemm_exact(x8, w8):
    """``acc[m, n] = sum_k dec(x8[m,k]) * dec(w8[n,k])`` exactly (float64).

    Runs in column blocks of at most 2048 outputs to bound memory."""
    X = e4m3_int(x8).astype(np.float64)
    M = X.shape[0]
    N = w8.shape[0]
    acc = np.empty((M, N), dtype=np.float64)
    for n0 in range(0, N, _COLS_PER_BLOCK):
        n1 = min(N, n0 + _COLS_PER_BLOCK)
        Wb = e4m3_int(w8[n0:n1]).astype(np.float64)
        acc[:, n0:n1] = X @ Wb.T
    return acc * _TWO_M18


def gemm_exact_at(x8, w8, rows, cols):
    """Exact ``acc`` at the sampled positions ``(rows[i], cols[i])`` only,
    each as its own K-length dot product of integer code values (int64:
    |k_x * k_w| < 2^36, so K <= 2^27 terms cannot overflow)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(rows.shape[0], dtype=np.float64)
    for lo in range(0, rows.shape[0], 256):
        hi = min(rows.shape[0], lo + 256)
        Xs = e4m3_int(x8[rows[lo:hi]])
        Ws = e4m3_int(w8[cols[lo:hi]])
        out[lo:hi] = (Xs * Ws).sum(axis=1).astype(np.float64)
    return out * _TWO_M18


def alpha_of(act_scale, w_scale):
    return np.float32(np.float32(act_scale) * np.float32(w_scale))


def epilogue(acc, act_scale, w_scale, bias_bits=None):
    """``alpha * acc + bias`` formed in float64 (no intermediate rounding)."""
    a = float(alpha_of(act_scale, w_scale))
    out = a * np.asarray(acc, dtype=np.float64)
    if bias_bits is not None:
        out = out + bf16_to_f32(bias_bits).astype(np.float64)
    return out


def to_bf16_ref(out64):
    """Round the exact epilogue to bf16 bits (via fp32: fp64 -> fp32 -> bf16
    can differ from a direct rounding only at a bf16 tie, within the one-ulp
    tolerance the comparison allows)."""
    return f32_to_bf16(np.asarray(out64, dtype=np.float64).astype(np.float32))


def split_columns(out, splits):
    """Sibling i takes columns ``[off_i, off_i + N_i)``."""
    res, off = [], 0
    for n in splits:
        res.append(out[:, off:off + n])
        off += n
    return res


def packed_gemm_split(x8, w8, act_scale, w_scale, bias_bits, splits):
    """Whole packed call: exact GEMM, epilogue, per-sibling outputs (fp64)."""
    out = epilogue(gemm_exact(x8, w8), act_scale, w_scale, bias_bits)
    return split_columns(out, splits)
