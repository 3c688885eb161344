"""Conditioned-norm producers and static FP8 activation quantisation.

Test infrastructure only (see the package docstring).

Sources (flashrt-structures 0.2.0 wheel pages):
- impls/adarms_stack/fp8_chain.py: the chain's per-layer producer call
  ``gate_residual_ada_norm_fp8_static_bf16(res, x, prev_gate, ones_w,
  style_row, act_scale, eps, out=xn8, gate_out=...)`` in ``_band_elements``;
  the chained residual in ``_make_run`` (``res.copy_(x)``, zero delta and
  gate before layer 0, the second site taking the first site's gate
  output); and the stack's fp32 tail, the only AdaRMS arithmetic the pages
  print: ``res = res + gate * delta``; ``res * rsqrt(mean(res^2) + eps)``;
  ``normed * (1 + fin[0]) + fin[1]``, where ``fin`` is the final norm's
  3D style row viewed as ``[3, D]``.
- impls/modnorm_qkv_chain/fp8_ptok_table.py: the per-token-table producer
  (module docstring: table add + chunk selection + no-affine LayerNorm +
  modulation + static FP8 quantize in one pass), the chunk roles
  ``(shift, scale, gate)`` = (0, 1, 2) attention / (3, 4, 5) FFN, the
  ``[6, D]`` fp32 table and ``[B*M, 6, D]`` bf16 temb layouts.
- the static activation scale: calibrated amax / 448 at the GEMM input
  (fp8_chain.py ``_quantize`` and the probe's forward pre-hooks); a site
  whose amax is not positive is refused.

Readings where the pages are silent:
- the norm runs on the fp32 gated residual, not on its bf16 rounding;
- the gated residual multiplies ``x`` by the *previous* site's gate (an
  input), and this row's gate chunk is only echoed to ``gate_out``;
- the 3D AdaRMS row is ``[scale | shift | gate]`` (the tail's ``fin[0]``
  scales, ``fin[1]`` shifts);
- the ptok modulation is the same ``y * (1 + scale) + shift``;
- y is not rounded to bf16 before quantisation; the quantiser divides
  ``y / act_scale`` in fp32 (the precision of the pages' own ``w.float() /
  scale``), clamps to +-448 and rounds to nearest even.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f32, f32_to_bf16, e4m3_encode, E4M3_MAX


def _bcast_rows(arr_bits, rows, D):
    """bf16 bits of shape [D] / [1, D] (one broadcast row) or [rows, D]."""
    a = bf16_to_f32(arr_bits)
    if a.ndim == 1:
        a = a[None, :]
    if a.shape[0] == 1 and rows != 1:
        a = np.broadcast_to(a, (rows, D))
    return a


def gated_residual(residual_bits, x_bits=None, gate_bits=None):
    """``h = residual + gate * x`` in fp32 and its bf16 write-back.

    (fp8_chain.py ``_make_run``: the in-place residual carried from site to
    site; the fp32 tail ``res.float() + gate.float() * delta.float()``.)

    The bf16 x bf16 product is exact in fp32 (8 + 8 significant bits), so
    ``h`` is the single fp32 rounding of the exact ``r + g*x``; NumPy's
    float32 multiply then add computes exactly that. ``x`` or ``gate``
    absent means a zero delta (layer 0 of the chain), so ``h = residual``.
    Returns ``(h_f32, residual_out_bits)``.
    """
    r = bf16_to_f32(residual_bits)
    rows, D = r.shape
    if x_bits is None or gate_bits is None:
        h = r.copy()
    else:
        x = bf16_to_f32(x_bits)
        g = _bcast_rows(gate_bits, rows, D)
        h = (r + (g * x).astype(np.float32)).astype(np.float32)
    return h, f32_to_bf16(h)


def ada_rms_norm(h_f32, mod_bits, eps, weight_bits=None):
    """AdaRMS of the fp32 residual ``h`` in fp64.

    ``y0 = h / sqrt(mean(h^2) + eps)`` (the stack tail's RMS step), then
    ``y = (y0 * w) * (1 + scale) + shift`` with the norm weight ``w`` (the
    chain passes ones) and ``scale, shift`` the first two D-chunks of the
    style row ``[scale | shift | gate]``. ``mod_bits`` is ``[1, 3D]``
    (one row broadcast to every token) or ``[rows, 3D]``. ``eps`` is used at
    its float32 value, the precision in which the kernel receives it.
    Returns ``y`` (float64, ``[rows, D]``).
    """
    h = np.asarray(h_f32, dtype=np.float64)
    rows, D = h.shape
    mod = _bcast_rows(mod_bits, rows, 3 * D).astype(np.float64)
    scale, shift = mod[:, 0:D], mod[:, D:2 * D]
    ms = np.mean(h * h, axis=1, keepdims=True)
    r = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    y0 = h * r
    if weight_bits is not None:
        y0 = y0 * bf16_to_f32(weight_bits).astype(np.float64)[None, :]
    return y0 * (1.0 + scale) + shift


def quantize_static(y, act_scale):
    """Static per-tensor FP8: ``e4m3(clamp(fl32(fl32(y) / s), -448, 448))``.

    The code is decided in fp32, as the pages' weight path does it
    (``(w.float() / scale).clamp(-448, 448).to(float8_e4m3fn)``): y is
    rounded to fp32, divided by the fp32 scale with one IEEE rounding,
    clamped and rounded to nearest even.
    """
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    q = (y32 / np.float32(act_scale)).astype(np.float32)
    return e4m3_encode(np.clip(q, -E4M3_MAX, E4M3_MAX))


def calibrate_act_scale(y_calib):
    """``fl32(fl32(amax) / 448)`` of the producer output on a calibration
    batch: the static scale measured at the GEMM input (fp8_chain.py
    ``_quantize``: ``amax / FP8_MAX``). A dead site (amax not positive) is
    refused, as the chain's bind refuses it."""
    amax = np.float32(np.max(np.abs(np.asarray(y_calib, dtype=np.float64))))
    if not amax > 0:
        raise ValueError("refused: calibration saw a dead quantizer site")
    return np.float32(amax / np.float32(E4M3_MAX))


def ada_norm_quant_fp8(residual_bits, x_bits, gate_bits, mod_bits,
                       act_scale, eps, weight_bits=None):
    """The gated-residual AdaRMS producer, end to end.

    Returns a dict with ``residual_out`` (bf16 bits), ``y`` (float64
    pre-quantisation output), ``codes`` (e4m3fn uint8) and ``gate_out``
    (the style row's gate chunk as bf16 bits, broadcast to every row).
    ``act_scale`` None skips the quantisation (calibration pass).
    """
    h, rout = gated_residual(residual_bits, x_bits, gate_bits)
    y = ada_rms_norm(h, mod_bits, eps, weight_bits)
    rows, D = h.shape
    mod = np.asarray(mod_bits, dtype=np.uint16).reshape(-1, 3 * D)
    gate_out = np.broadcast_to(mod[:, 2 * D:3 * D], (rows, D)).copy()
    out = {"residual_out": rout, "y": y, "h": h, "gate_out": gate_out}
    if act_scale is not None:
        out["codes"] = quantize_static(y, act_scale)
    return out


def ptok_layer_norm(x_bits, temb_bits, table, shift_idx, scale_idx, eps):
    """Per-token-table no-affine adaptive LayerNorm in fp64.

    Per row r: ``shift = fl32(table[s] + temb[r, s])``,
    ``scale = fl32(table[c] + temb[r, c])`` (fp32 table plus bf16 temb, the
    sum the producer forms in fp32); ``mu = mean(x)``,
    ``var = mean((x - mu)^2)`` (biased, two-pass);
    ``y = (x - mu) / sqrt(var + eps) * (1 + scale) + shift``.
    ``temb`` is ``[R, C, D]`` with row r paired with x row r.
    """
    x = bf16_to_f32(x_bits).astype(np.float64)
    R, D = x.shape
    t = np.asarray(temb_bits, dtype=np.uint16).reshape(R, -1, D)
    tab = np.asarray(table, dtype=np.float32)
    shift = (tab[shift_idx][None, :] + bf16_to_f32(t[:, shift_idx, :])
             ).astype(np.float32).astype(np.float64)
    scale = (tab[scale_idx][None, :] + bf16_to_f32(t[:, scale_idx, :])
             ).astype(np.float32).astype(np.float64)
    mu = np.mean(x, axis=1, keepdims=True)
    d = x - mu
    var = np.mean(d * d, axis=1, keepdims=True)
    xn = d / np.sqrt(var + float(np.float32(eps)))
    return xn * (1.0 + scale) + shift


def ptok_norm_quant_fp8(x_bits, temb_bits, table, act_scale, shift_idx,
                        scale_idx, eps):
    """The per-token-table producer end to end: ``{"y", "codes"}``."""
    y = ptok_layer_norm(x_bits, temb_bits, table, shift_idx, scale_idx, eps)
    out = {"y": y}
    if act_scale is not None:
        out["codes"] = quantize_static(y, act_scale)
    return out
