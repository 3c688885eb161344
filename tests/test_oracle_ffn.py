"""Pins for the oracle's GEGLU quantiser and the merged gate/up composition
(CPU only).

``gelu_tanh`` is pinned to torch's own tanh-GELU (an independent library
implementation), to the odd-part identity ``gelu(v) - gelu(-v) = v`` that the
tanh form satisfies exactly in real arithmetic, to its limits, and to the
exact (erf) GELU within the approximation's small error. The GEGLU halves are
pinned by reductions that tell gate from up. The whole gate/up -> GEGLU ->
FP8 chain is pinned to a brute-force evaluation on a tiny case (exact
rational GEMM, torch's bf16 and float8 casts, ``math.tanh``).
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, ffn, producers
from workloads import random_codes, to_bf16_bits


def _bf(a):
    return to_bf16_bits(np.asarray(a, np.float32))


def test_gelu_tanh_matches_torch():
    rng = np.random.default_rng(31)
    v = np.concatenate([rng.standard_normal(100000) * 3.0,
                        np.linspace(-12, 12, 4001),
                        [0.0, -0.0, 1e-30, -1e-30, 40.0, -40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    got = ffn.gelu_tanh(v)
    err = np.abs(got - ref)
    assert np.all(err <= 4e-16 * np.maximum(np.abs(ref), 1.0))
    # and it is not the erf form, which differs by up to ~1e-3
    erf_form = torch.nn.functional.gelu(torch.from_numpy(v)).numpy()
    assert np.max(np.abs(got - erf_form)) > 1e-4


def test_gelu_tanh_identities_and_limits():
    v = np.linspace(-9, 9, 2001)
    # 0.5 v (1 + tanh z) - 0.5 (-v)(1 - tanh z) = v
    assert np.allclose(ffn.gelu_tanh(v) - ffn.gelu_tanh(-v), v, rtol=0, atol=1e-14)
    assert ffn.gelu_tanh(np.array([0.0]))[0] == 0.0
    # slope 1/2 at zero
    h = 1e-6
    d = (ffn.gelu_tanh(np.array([h])) - ffn.gelu_tanh(np.array([-h])))[0] / (2 * h)
    assert abs(d - 0.5) < 1e-9
    assert ffn.gelu_tanh(np.array([30.0]))[0] == 30.0
    assert ffn.gelu_tanh(np.array([-30.0]))[0] == 0.0
    # tracks the exact GELU v * Phi(v) within the tanh form's known error
    exact = np.array([x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) for x in v])
    assert np.max(np.abs(ffn.gelu_tanh(v) - exact)) < 5e-4


def test_geglu_takes_gate_from_the_first_half():
    rng = np.random.default_rng(32)
    M, H = 4, 96
    g = _bf(rng.standard_normal((M, H)) * 2)
    ones = _bf(np.ones((M, H)))
    # up = 1: y = gelu(gate)
    y = ffn.geglu(np.concatenate([g, ones], axis=1), H)
    assert np.array_equal(y, ffn.gelu_tanh(codecs.bf16_to_f32(g).astype(np.float64)))
    # gate = 1 instead: y = gelu(1) * up, not gelu(up)
    y2 = ffn.geglu(np.concatenate([ones, g], axis=1), H)
    assert np.allclose(y2, ffn.gelu_tanh(np.array([1.0]))[0] * codecs.bf16_to_f32(g), rtol=1e-15)
    # columns past 2H (a wider row stride) are ignored
    extra = _bf(rng.standard_normal((M, 8)))
    y3 = ffn.geglu(np.concatenate([g, ones, extra], axis=1), H)
    assert np.array_equal(y3, y)


def test_geglu_quant_invariants():
    rng = np.random.default_rng(33)
    M, H = 8, 512
    gu = _bf(rng.standard_normal((M, 2 * H)) * 3)
    y = ffn.geglu(gu, H)
    s = producers.calibrate_act_scale(y)
    r = ffn.geglu_quant_fp8(gu, H, s)
    c = r["codes"]
    dec = codecs.e4m3_decode(c).astype(np.float64)
    assert np.all(np.isfinite(dec))
    # the largest |y| lands on (or next to) the top code
    assert np.max(np.abs(dec)) >= 416.0
    # half a quantisation step, judged at the code's own binade
    step = np.where(np.abs(dec) >= 2.0 ** -6,
                    2.0 ** (np.floor(np.log2(np.maximum(np.abs(dec), 2.0 ** -6))) - 3),
                    2.0 ** -9)
    assert np.all(np.abs(dec * float(s) - y) <= 0.5 * step * float(s) * (1 + 1e-6) + 1e-12)
    # saturation: a scale 100x too small clamps to +-448, never NaN
    c_sat = ffn.geglu_quant_fp8(gu, H, np.float32(s / 100))["codes"]
    d_sat = codecs.e4m3_decode(c_sat)
    assert np.all(np.isfinite(d_sat)) and np.max(np.abs(d_sat)) == 448.0


def _brute_chain(x8, w8, H, s_a, s_w, s_o):
    """Tiny-case brute force of GEMM -> bf16 -> GEGLU -> FP8, written with
    Fraction, math.tanh and torch's casts (none of the oracle's helpers)."""
    def dec(c):
        return Fraction(float(torch.tensor([int(c)], dtype=torch.uint8)
                              .view(torch.float8_e4m3fn).float().item()))

    M, K = x8.shape
    alpha = float(np.float32(np.float32(s_a) * np.float32(s_w)))
    gu = np.zeros((M, 2 * H))
    for m in range(M):
        for n in range(2 * H):
            acc = sum((dec(x8[m, k]) * dec(w8[n, k]) for k in range(K)), Fraction(0))
            v = float(np.float32(alpha * float(acc)))
            gu[m, n] = torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float().item()
    codes = np.zeros((M, H), np.uint8)
    c = math.sqrt(2.0 / math.pi)
    for m in range(M):
        for j in range(H):
            g, u = gu[m, j], gu[m, H + j]
            y = 0.5 * g * (1.0 + math.tanh(c * (g + 0.044715 * g ** 3))) * u
            q = np.float32(np.float32(y) / np.float32(s_o))
            t = torch.tensor([float(q)], dtype=torch.float32).clamp(-448, 448)
            codes[m, j] = t.to(torch.float8_e4m3fn).view(torch.uint8).item()
    return gu, codes


def test_gate_up_chain_brute_force():
    M, K, H = 3, 64, 5
    x8 = random_codes(41, (M, K))
    w8 = random_codes(42, (2 * H, K))
    s_a, s_w, s_o = np.float32(0.013), np.float32(0.0021), np.float32(2e-3)
    gu_ref, codes_ref = _brute_chain(x8, w8, H, s_a, s_w, s_o)
    r = ffn.gate_up_gelu_quant(x8, w8, H, s_a, s_w, None, s_o)
    assert np.array_equal(codecs.bf16_to_f32(r["gu"]), gu_ref.astype(np.float32))
    assert np.array_equal(r["codes"], codes_ref)


def test_gate_up_chain_rejects_odd_weight():
    with pytest.raises(ValueError):
        ffn.gate_up_gelu_quant(random_codes(1, (2, 64)), random_codes(2, (7, 64)),
                               4, 1.0, 1.0, None, 1.0)
