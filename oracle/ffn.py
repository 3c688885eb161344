"""GEGLU + static FP8 quantisation of the merged gate/up output, and the
gate/up GEMM that produces it.

Test infrastructure only (see the package docstring).

Sources (flashrt-structures 0.2.0 wheel pages):
- impls/adarms_stack/fp8_chain.py ``_quantize``: the FFN's gate and up
  projections are packed as one matrix, gate rows first
  (``cat([gate_proj.weight, up_proj.weight])``), so the merged GEMM output
  ``gu`` (``[S, 2H]`` bf16, allocated in ``_alloc``) holds the gate in
  columns ``[0, H)`` and up in ``[H, 2H)``;
- the same page's ``_band_elements`` (``down_project``): the fused
  ``gate_geglu_merged_quant_fp8_static_bf16(gu, t_sc_dn, out=hid8)`` writes
  the FP8 ``[S, H]`` input of the down projection, which is then the plain
  static FP8 linear ``fp8_linear_bf16(hid8, dn, alpha=a_dn)`` (the packed
  GEMM of ``oracle.gemm`` with one sibling and no bias);
- the chain's bind refuses a stack whose FFN activation is not tanh-GELU.

Readings where the pages are silent:
- GEGLU is ``act(gate) * up`` with ``act`` the tanh form of GELU,
  ``0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))`` -- the host MLP
  ``down(act(gate(x)) * up(x))`` that the merged GEMM feeds;
- gate and up enter as the bf16 values the merged GEMM writes, so a fused
  form must round its fp32 accumulator to bf16 first, as the unfused GEMM
  output is rounded;
- ``y = act(g) * u`` is formed in fp64 and quantised like every static
  site (``oracle.producers.quantize_static``): ``fl32(fl32(y) / s)``,
  clamped to +-448, rounded to nearest even;
- the down projection's activation scale is calibrated like the other
  sites: amax of ``y`` on the calibration batch, over 448.
"""

from __future__ import annotations

import math

import numpy as np

from .codecs import bf16_to_f32
from .gemm import epilogue, gemm_exact, to_bf16_ref
from .producers import quantize_static

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_CUBIC = 0.044715


def gelu_tanh(v):
    """Tanh-approximated GELU in float64:
    ``0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))``."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(_SQRT_2_OVER_PI * (v + _CUBIC * v * v * v)))


def geglu(gu_bits, H):
    """``y[m, j] = gelu_tanh(gate[m, j]) * up[m, j]`` in float64, with
    ``gate = gu[:, :H]`` and ``up = gu[:, H:2H]`` decoded from bf16."""
    gu = bf16_to_f32(np.asarray(gu_bits, dtype=np.uint16)).astype(np.float64)
    if gu.ndim != 2 or gu.shape[1] < 2 * H:
        raise ValueError("gu must be [M, >= 2H]")
    return gelu_tanh(gu[:, :H]) * gu[:, H:2 * H]


def geglu_quant_fp8(gu_bits, H, act_scale):
    """The merged GEGLU + static FP8 quantiser: ``{"y", "codes"}``;
    ``act_scale`` None skips the quantisation (calibration pass)."""
    y = geglu(gu_bits, H)
    out = {"y": y}
    if act_scale is not None:
        out["codes"] = quantize_static(y, act_scale)
    return out


def gate_up_gelu_quant(x8, w8_gu, H, act_scale, w_scale, bias_bits,
                       out_scale):
    """The merged gate/up GEMM followed by the GEGLU quantiser, as the pages
    chain them: exact GEMM, ``alpha * acc + bias`` rounded once to bf16 (the
    ``gu`` buffer), then ``geglu_quant_fp8``. ``w8_gu`` is ``[2H, K]`` with
    the gate rows first. Returns ``{"gu", "y", "codes"}``."""
    w8_gu = np.asarray(w8_gu)
    if w8_gu.shape[0] != 2 * H:
        raise ValueError("w8_gu must hold 2H rows")
    gu = to_bf16_ref(epilogue(gemm_exact(x8, w8_gu), act_scale, w_scale,
                              bias_bits))
    r = geglu_quant_fp8(gu, H, out_scale)
    r["gu"] = gu
    return r
