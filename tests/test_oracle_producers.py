"""Pins for the oracle's producers (CPU only): closed forms, special cases
that reduce to torch CPU library routines (rms_norm, layer_norm), and
invariants of the static quantiser."""

import numpy as np
import pytest
import torch

from oracle import codecs, producers
from workloads import to_bf16_bits

EPS = 1e-6
EPS32 = float(np.float32(EPS))


def _bf(a):
    return to_bf16_bits(np.asarray(a, np.float32))


def _mod(scale, shift, gate, D):
    row = np.concatenate([np.broadcast_to(np.float32(scale), (D,)),
                          np.broadcast_to(np.float32(shift), (D,)),
                          np.broadcast_to(np.float32(gate), (D,))])
    return _bf(row[None, :])


# -------------------------------------------------------------- gated residual

def test_gated_residual_exact_single_rounding():
    rng = np.random.default_rng(1)
    rows, D = 8, 512
    r, x, g = (_bf(rng.standard_normal((rows, D)) * s) for s in (1, 1, 0.5))
    h, rout = producers.gated_residual(r, x, g)
    # the exact sum in rationals, rounded once to fp32
    R, X, G = (codecs.bf16_to_f32(a).astype(np.float64) for a in (r, x, g))
    exact = R + G * X        # exact in fp64 at these magnitudes
    assert np.array_equal(h, exact.astype(np.float32))
    assert np.array_equal(rout, codecs.f32_to_bf16(h))


def test_gated_residual_zero_gate_is_identity():
    rng = np.random.default_rng(2)
    r = _bf(rng.standard_normal((4, 512)))
    x = _bf(rng.standard_normal((4, 512)))
    zero = np.zeros(512, np.uint16)
    h, rout = producers.gated_residual(r, x, zero)
    assert np.array_equal(rout, r)
    h2, rout2 = producers.gated_residual(r, None, None)
    assert np.array_equal(rout2, r) and np.array_equal(h, h2)


def test_gated_residual_broadcast_row_equals_full_rows():
    rng = np.random.default_rng(3)
    r = _bf(rng.standard_normal((5, 512)))
    x = _bf(rng.standard_normal((5, 512)))
    g = _bf(rng.standard_normal(512) * 0.1)
    h1, _ = producers.gated_residual(r, x, g)
    h2, _ = producers.gated_residual(r, x, np.tile(g, (5, 1)))
    assert np.array_equal(h1, h2)


# -------------------------------------------------------------- AdaRMS

@pytest.mark.parametrize("c", [1e-3, 0.5, 3.0, -7.25])
def test_adarms_constant_row_closed_form(c):
    D = 512
    h = np.full((1, D), np.float32(c), np.float32)
    a, b = np.float32(0.25), np.float32(-0.375)     # exact in bf16
    y = producers.ada_rms_norm(h, _mod(a, b, 0.0, D), EPS)
    c64 = float(np.float32(c))
    want = c64 / np.sqrt(c64 * c64 + EPS32) * (1 + 0.25) - 0.375
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=0)


def test_adarms_scale_minus_one_gives_shift():
    rng = np.random.default_rng(4)
    D = 768
    h = rng.standard_normal((3, D)).astype(np.float32)
    shift = rng.standard_normal(D).astype(np.float32) * 0.1
    mod = _bf(np.concatenate([-np.ones(D, np.float32), shift,
                              np.zeros(D, np.float32)])[None, :])
    y = producers.ada_rms_norm(h, mod, EPS)
    want = codecs.bf16_to_f32(mod[0, D:2 * D]).astype(np.float64)
    assert np.array_equal(y, np.broadcast_to(want, y.shape))


def test_adarms_zero_row_gives_shift():
    D = 512
    y = producers.ada_rms_norm(np.zeros((2, D), np.float32),
                               _mod(0.5, 0.125, 0.0, D), EPS)
    assert np.array_equal(y, np.full((2, D), 0.125))


def test_adarms_plain_rmsnorm_matches_torch():
    rng = np.random.default_rng(5)
    D = 1024
    h = (rng.standard_normal((16, D)) * 3).astype(np.float32)
    w = _bf(rng.standard_normal(D) * 0.5 + 1)
    y = producers.ada_rms_norm(h, _mod(0.0, 0.0, 0.0, D), EPS, weight_bits=w)
    ref = torch.nn.functional.rms_norm(
        torch.from_numpy(h.astype(np.float64)), (D,),
        weight=torch.from_numpy(codecs.bf16_to_f32(w).astype(np.float64)),
        eps=EPS32).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_adarms_modulation_chunk_order():
    """[scale | shift | gate]: distinct per-chunk values must land in their
    own roles (a swapped or shifted chunk index fails)."""
    D = 512
    rng = np.random.default_rng(6)
    h = rng.standard_normal((4, D)).astype(np.float32)
    scale = np.linspace(-0.5, 0.5, D).astype(np.float32)
    shift = np.linspace(1.0, 2.0, D).astype(np.float32)
    gate = np.full(D, 9.0, np.float32)
    mod = _bf(np.concatenate([scale, shift, gate])[None, :])
    y = producers.ada_rms_norm(h, mod, EPS)
    h64 = h.astype(np.float64)
    r = 1 / np.sqrt((h64 ** 2).mean(1, keepdims=True) + EPS32)
    sc = codecs.bf16_to_f32(mod[0, :D]).astype(np.float64)
    sh = codecs.bf16_to_f32(mod[0, D:2 * D]).astype(np.float64)
    np.testing.assert_allclose(y, h64 * r * (1 + sc) + sh, rtol=1e-13,
                               atol=1e-13)
    out = producers.ada_norm_quant_fp8(_bf(h), None, None, mod, None, EPS)
    assert np.array_equal(out["gate_out"], np.tile(mod[0, 2 * D:], (4, 1)))


def test_adarms_eps_matters():
    """A dropped or misplaced eps fails: at |h| ~ 1e-3 eps is half the
    mean square."""
    D = 512
    h = np.full((1, D), np.float32(1e-3), np.float32)
    y = producers.ada_rms_norm(h, _mod(0, 0, 0, D), EPS)
    c = float(np.float32(1e-3))
    assert abs(y[0, 0] - c / np.sqrt(c * c + EPS32)) < 1e-12
    assert abs(y[0, 0] - 1.0) > 0.1


# -------------------------------------------------------------- ptok LayerNorm

def _ptok_inputs(R, D, seed, tab_std=0.1, temb_std=0.1):
    rng = np.random.default_rng(seed)
    x = _bf(rng.standard_normal((R, D)))
    temb = _bf(rng.standard_normal((R, 6, D)) * temb_std)
    table = (rng.standard_normal((6, D)) * tab_std).astype(np.float32)
    return x, temb, table


def test_ptok_no_modulation_matches_torch_layer_norm():
    R, D = 8, 1024
    x, temb, table = _ptok_inputs(R, D, 7)
    # table = -temb (in fp32) makes shift = scale = 0 exactly
    t32 = codecs.bf16_to_f32(temb)
    zero_table = np.zeros((6, D), np.float32)
    temb0 = np.zeros_like(temb)
    y = producers.ptok_layer_norm(x, temb0, zero_table, 0, 1, EPS)
    ref = torch.nn.functional.layer_norm(
        torch.from_numpy(codecs.bf16_to_f32(x).astype(np.float64)), (D,),
        eps=EPS32).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s_idx,c_idx", [(0, 1), (3, 4)])
def test_ptok_chunk_selection_and_modulation(s_idx, c_idx):
    R, D = 6, 512
    x, temb, table = _ptok_inputs(R, D, 8)
    y = producers.ptok_layer_norm(x, temb, table, s_idx, c_idx, EPS)
    X = codecs.bf16_to_f32(x).astype(np.float64)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(X), (D,),
                                        eps=EPS32).numpy()
    T = codecs.bf16_to_f32(temb)
    sh = (table[s_idx][None] + T[:, s_idx]).astype(np.float64)
    sc = (table[c_idx][None] + T[:, c_idx]).astype(np.float64)
    np.testing.assert_allclose(y, ln * (1 + sc) + sh, rtol=1e-10, atol=1e-10)


def test_ptok_constant_row_gives_shift():
    R, D = 3, 512
    _, temb, table = _ptok_inputs(R, D, 9)
    x = _bf(np.full((R, D), 2.5, np.float32))
    y = producers.ptok_layer_norm(x, temb, table, 3, 4, EPS)
    T = codecs.bf16_to_f32(temb)
    want = (table[3][None] + T[:, 3]).astype(np.float32).astype(np.float64)
    assert np.array_equal(y, want)


def test_ptok_two_value_row_closed_form():
    D = 512
    a, b = 1.5, -0.25
    row = np.where(np.arange(D) % 2 == 0, a, b).astype(np.float32)
    x = _bf(row[None, :])
    temb = np.zeros((1, 6, D), np.uint16)
    y = producers.ptok_layer_norm(x, temb, np.zeros((6, D), np.float32), 0,
                                  1, EPS)
    half = (a - b) / 2
    want = np.where(np.arange(D) % 2 == 0, half, -half) / np.sqrt(
        half * half + EPS32)
    np.testing.assert_allclose(y[0], want, rtol=1e-14)


# -------------------------------------------------------------- quantiser

def test_quantize_invariants():
    rng = np.random.default_rng(10)
    y = rng.standard_normal(200_000) * np.exp(rng.uniform(-6, 3, 200_000))
    s = np.float32(0.0123)
    q = producers.quantize_static(y, s)
    ordv = codecs.e4m3_ordinal(q)
    assert np.all((q & 0x7F) != 0x7F)                    # no NaN
    dec = codecs.e4m3_decode(q)
    assert np.all(np.abs(dec) <= 448)
    inside = np.abs(y) <= 448 * float(s)
    # half a step of the nearest code, at the code's own exponent
    mags = codecs.E4M3_VALUES[:0x7F]
    step = np.diff(mags)
    idx = np.abs(ordv[inside])
    ulp = np.maximum(step[np.minimum(idx, 125)], step[np.maximum(idx - 1, 0)])
    err = np.abs(dec[inside] * float(s) - y[inside])
    assert np.all(err <= 0.5 * ulp * float(s) * (1 + 1e-6))
    # saturation outside the range
    assert np.all(q[y > 448 * float(s) * 1.01] == 0x7E)
    assert np.all(q[y < -448 * float(s) * 1.01] == 0xFE)


def test_quantize_decides_in_fp32():
    """The code follows the fp32 quotient: a y whose fp64 quotient sits just
    below a midpoint but whose fp32 quotient lands on it rounds as a tie."""
    s = np.float32(1.0)
    mid = 1.0625                     # midpoint between 1.0 and 1.125
    y = mid - 2.0 ** -40             # rounds to the midpoint in fp32
    assert np.float32(y) == np.float32(mid)
    assert producers.quantize_static(np.array([y]), s)[0] == 0x38


def test_calibration_scale_and_dead_site():
    y = np.array([[0.5, -2.0, 1.0]])
    assert producers.calibrate_act_scale(y) == np.float32(np.float32(2.0) / 448)
    with pytest.raises(ValueError, match="dead"):
        producers.calibrate_act_scale(np.zeros((2, 3)))


def test_ada_norm_quant_end_to_end_codes_consistent():
    rng = np.random.default_rng(11)
    D = 512
    r, x = (_bf(rng.standard_normal((4, D))) for _ in range(2))
    g = _bf(rng.standard_normal(D) * 0.1)
    mod = _bf(rng.standard_normal((1, 3 * D)) * 0.1)
    cal = producers.ada_norm_quant_fp8(r, x, g, mod, None, EPS)
    s = producers.calibrate_act_scale(cal["y"])
    out = producers.ada_norm_quant_fp8(r, x, g, mod, s, EPS)
    # the calibration batch itself never saturates and uses the top code
    assert np.abs(codecs.e4m3_ordinal(out["codes"])).max() == 126
