"""GPU parity of the FFN tail: the GEGLU quantiser of the merged gate/up
output (standalone), the gate/up GEMM with the GEGLU quantiser as its
epilogue, and the down projection that consumes the codes, against the
oracle, through the C ABI.

Rules (see gpu_util): codes within one e4m3 step on at most 0.1 % of the
elements; y rows within 1e-5 of the oracle's fp64 y.

The fused GEMM is checked in three links, each against what decides it:
- its codes equal, bit for bit, those of the unfused chain on the GPU (the
  split GEMM's bf16 gate|up output fed to the standalone quantiser): both
  round the same fp32 accumulators to bf16 and run the same GEGLU
  arithmetic;
- that bf16 gate|up output is within the GEMM tolerance of the exact
  oracle GEMM;
- the codes are within the code tolerance of the oracle's GEGLU quantiser
  applied to that bf16 output. (Against the all-oracle chain the codes can
  differ more often: the matrix cores' fp32 accumulation is ~1e-4 of
  max|acc| from exact, enough to flip a bf16 rounding of gate or up now and
  then, and the code with it; the code is decided from the bf16 values, so
  that is where it is compared.)
"""

import numpy as np
import pytest
import torch

import norm_quantize_packed_amd as frt
import workloads as wl
from oracle import codecs, ffn, gemm, pack, producers
from gpu_util import (Guarded, assert_codes_close, assert_codes_quantise_own_y,
                      assert_gemm_bf16, assert_rows_close, dev_bf16, dev_u8,
                      host_bf16, host_u8, scalar)

pytestmark = pytest.mark.gpu


def _gu_bits(seed, M, width, std=2.0):
    return wl.random_bf16(seed, (M, width), std)


@pytest.mark.parametrize("M,H,extra", [(1, 8, 0), (7, 1024, 0), (5, 1000, 8),
                                       (3, 1001, 3), (33, 136, 24),
                                       (256, 8192, 0)])
def test_geglu_quant_vs_oracle(M, H, extra):
    gu = _gu_bits(100 + H, M, 2 * H + extra)
    ref = ffn.geglu(gu, H)
    s = producers.calibrate_act_scale(ref)
    codes_ref = ffn.geglu_quant_fp8(gu, H, s)["codes"]
    out = Guarded(M, H, torch.uint8, ld=H + (extra // 2) * 2)
    y = Guarded(M, H, torch.float32, ld=H + extra)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    frt.frt_geglu_quant_fp8(dev_bf16(gu), H, scalar(s), out_fp8=out.view,
                            y_f32=y.view, amax_out=amax)
    torch.cuda.synchronize()
    out.check_guards()
    y.check_guards()
    got_y = y.view.cpu().numpy()
    got = host_u8(out.view)
    assert_rows_close(got_y, ref, what=f"geglu y {M}x{H}")
    assert_codes_close(got, codes_ref, what=f"geglu codes {M}x{H}")
    assert_codes_quantise_own_y(got, got_y, s)
    assert amax.item() == np.float32(np.max(np.abs(got_y)))


def test_geglu_rows_beyond_M_untouched_and_empty():
    H = 512
    gu = _gu_bits(7, 8, 2 * H)
    out = torch.full((8, H), 0x5A, dtype=torch.uint8, device="cuda")
    frt.frt_geglu_quant_fp8(dev_bf16(gu), H, scalar(0.01), out_fp8=out, M=5)
    frt.frt_geglu_quant_fp8(dev_bf16(gu), H, scalar(0.01), out_fp8=out[5:], M=0)
    torch.cuda.synchronize()
    o = host_u8(out)
    assert (o[5:] == 0x5A).all()
    ref = ffn.geglu_quant_fp8(gu[:5], H, np.float32(0.01))["codes"]
    assert_codes_close(o[:5], ref, what="geglu M=5")


def test_geglu_saturates_and_keeps_signs():
    """Huge products clamp to +-448 (codes 0x7E / 0xFE), never NaN; the
    negative tail of GELU gives -0-ish codes, not garbage."""
    H = 64
    v = np.zeros((2, 2 * H), np.float32)
    v[0, :H] = np.linspace(-20, 20, H)
    v[0, H:] = 1e4
    v[1, :H] = -30.0
    v[1, H:] = np.linspace(-3, 3, H)
    gu = wl.to_bf16_bits(v)
    out = torch.empty((2, H), dtype=torch.uint8, device="cuda")
    frt.frt_geglu_quant_fp8(dev_bf16(gu), H, scalar(1.0), out_fp8=out)
    torch.cuda.synchronize()
    got = host_u8(out)
    ref = ffn.geglu_quant_fp8(gu, H, np.float32(1.0))["codes"]
    d = np.abs(codecs.e4m3_ordinal(got) - codecs.e4m3_ordinal(ref))
    assert d.max() <= 1
    assert (got[0, H // 2 + 4:] == 0x7E).all()     # gelu(g) * 9984 > 448
    dec = codecs.e4m3_decode(got)
    assert np.all(np.isfinite(dec)) and dec.max() == 448.0


# ------------------------------------------------ fused gate/up + GEGLU GEMM

def _operands(M, K, H, seed, bias=False, w_std=0.02):
    """FP8 activations (a calibrated N(0,1) batch) and a packed [gate; up]
    weight, both from the oracle's own quantiser and packer."""
    x = wl.random_bf16(seed, (M, K), 1.0)
    xf = codecs.bf16_to_f32(x).astype(np.float64)
    s_a = producers.calibrate_act_scale(xf)
    x8 = producers.quantize_static(xf, s_a)
    Wg = wl.random_bf16(seed + 1, (H, K), w_std)
    Wu = wl.random_bf16(seed + 2, (H, K), w_std)
    bs = [wl.random_bf16(seed + 3, (H,), 0.02), wl.random_bf16(seed + 4, (H,), 0.02)] if bias else None
    w8, s_w, bias_cat, _ = pack.pack_weights([Wg, Wu], bs)
    return x8, s_a, w8, s_w, (bias_cat if bias else None)


def _run_fused(x8, s_a, w8, s_w, bias, s_o, H, M=None, ld_out=None):
    Mv = x8.shape[0] if M is None else M
    out = Guarded(Mv, H, torch.uint8, ld=ld_out)
    frt.frt_packed_gemm_fp8_geglu_quant(
        dev_u8(x8), dev_u8(w8), scalar(s_a), scalar(s_w), scalar(s_o), out.view,
        None if bias is None else dev_bf16(bias), M=Mv)
    torch.cuda.synchronize()
    out.check_guards()
    return host_u8(out.view)


def _run_unfused(x8, s_a, w8, s_w, bias, s_o, H, M=None):
    """The split GEMM's bf16 gate|up output and the standalone quantiser's
    codes of it: (codes, gu bf16 bits)."""
    Mv = x8.shape[0] if M is None else M
    gu = torch.empty((Mv, 2 * H), dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_fp8_split(dev_u8(x8), dev_u8(w8), scalar(s_a), scalar(s_w), [gu],
                                  [2 * H], None if bias is None else dev_bf16(bias), M=Mv)
    codes = torch.empty((Mv, H), dtype=torch.uint8, device="cuda")
    frt.frt_geglu_quant_fp8(gu, H, scalar(s_o), out_fp8=codes)
    torch.cuda.synchronize()
    return host_u8(codes), host_bf16(gu)


@pytest.mark.parametrize("M,K,H,bias", [
    (1, 512, 256, False),     # small-M plan, one row
    (16, 1024, 200, True),    # ragged H (last tile half empty), bias
    (64, 1040, 320, False),   # K tail (K % 128 != 0)
    (65, 2048, 1024, False),  # mid-M plan with too few tiles -> 64x64
    (256, 2048, 8192, False), # the decoder layer's gate/up (128x128 plan)
    (600, 1536, 704, True),   # M >= 512 (64x64 plan: least per-CU load), ragged M and H
    (2000, 6160, 2500, True), # deep-K 256x256 plan (four 128x128 waves), ragged M, H, K
    (2000, 2064, 2500, False), # deep-K plan near its K threshold, K tail
])
def test_gemm_geglu_vs_oracle_and_unfused(M, K, H, bias):
    x8, s_a, w8, s_w, bc = _operands(M, K, H, 500 + M, bias)
    y = ffn.gate_up_gelu_quant(x8, w8, H, s_a, s_w, bc, None)["y"]
    s_o = producers.calibrate_act_scale(y)
    got = _run_fused(x8, s_a, w8, s_w, bc, s_o, H, ld_out=H + 16)
    unf, gu = _run_unfused(x8, s_a, w8, s_w, bc, s_o, H)
    assert np.array_equal(got, unf)
    exact = gemm.epilogue(gemm.gemm_exact(x8, w8), s_a, s_w, bc)
    assert_gemm_bf16(gu, exact, what=f"gate|up {M}x{2 * H}x{K}")
    ref = ffn.geglu_quant_fp8(gu, H, s_o)["codes"]
    assert_codes_close(got, ref, what=f"fused {M}x{2 * H}x{K}")


def test_gemm_geglu_row_capacity():
    """M below the buffer's rows: only M rows are written (guards around the
    logical region), the rest of a larger buffer stays untouched."""
    M, K, H = 40, 1024, 512
    x8, s_a, w8, s_w, _ = _operands(64, K, H, 77)
    out = torch.full((64, H), 0x33, dtype=torch.uint8, device="cuda")
    frt.frt_packed_gemm_fp8_geglu_quant(dev_u8(x8), dev_u8(w8), scalar(s_a), scalar(s_w),
                                        scalar(0.05), out, M=M)
    torch.cuda.synchronize()
    o = host_u8(out)
    assert (o[M:] == 0x33).all()
    unf, gu = _run_unfused(x8, s_a, w8, s_w, None, np.float32(0.05), H, M=M)
    assert np.array_equal(o[:M], unf)
    ref = ffn.geglu_quant_fp8(gu, H, np.float32(0.05))["codes"]
    assert_codes_close(o[:M], ref, what="fused M=40")


def test_gemm_geglu_widest_workload_sampled():
    """The 2048-token DiT FFN shape (gate|up 16384|16384 over K = 16384, the
    256x256 plan over a full chip of tiles): sampled codes against the
    oracle (exact dot products at the sampled positions), and every code
    equal to the unfused chain's."""
    M, K, H = 2048, 16384, 16384
    rng = np.random.default_rng(9)

    def codes(shape, top):
        # e4m3 codes uniform over magnitudes [0, top) with a random sign
        # (top 0x50: |x| < 8; top 0x40: |w| < 2)
        mag = rng.integers(0, top, size=shape, dtype=np.uint8)
        return mag | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)

    x8 = codes((M, K), 0x50)
    w8 = codes((2 * H, K), 0x40)
    s_a, s_w = np.float32(0.01), np.float32(0.004)
    rows = rng.integers(0, M, 1024)
    cols = rng.integers(0, H, 1024)
    g = gemm.epilogue(gemm.gemm_exact_at(x8, w8, rows, cols), s_a, s_w)
    u = gemm.epilogue(gemm.gemm_exact_at(x8, w8, rows, cols + H), s_a, s_w)
    y = ffn.geglu(np.stack([gemm.to_bf16_ref(g), gemm.to_bf16_ref(u)], axis=1), 1)[:, 0]
    s_o = np.float32(np.float32(np.max(np.abs(y)) * 1.5) / np.float32(448))
    got = _run_fused(x8, s_a, w8, s_w, None, s_o, H)
    unf, gu = _run_unfused(x8, s_a, w8, s_w, None, s_o, H)
    assert np.array_equal(got, unf)
    # the sampled gate and up values within the GEMM tolerance of exact
    scale = max(np.max(np.abs(g)), np.max(np.abs(u)))
    assert_gemm_bf16(gu[rows, cols], g, what="gate sampled", scale=scale)
    assert_gemm_bf16(gu[rows, cols + H], u, what="up sampled", scale=scale)
    pair = np.stack([gu[rows, cols], gu[rows, cols + H]], axis=1)
    ref = ffn.geglu_quant_fp8(pair, 1, s_o)["codes"][:, 0]
    assert_codes_close(got[rows, cols], ref, what="fused 2048x32768x16384 sampled")


def test_down_projection_vs_oracle():
    """The FFN's down projection on the GEGLU codes (decoder layer: 256 x
    2048 x 8192, one sibling, no bias), bf16 out."""
    M, H = 256, 8192
    D = wl.WORKLOADS[2].D
    x8, s_a, w8, s_w, _ = _operands(M, D, H, 300)
    r = ffn.gate_up_gelu_quant(x8, w8, H, s_a, s_w, None, None)
    s_h = producers.calibrate_act_scale(r["y"])
    hid8 = producers.quantize_static(r["y"], s_h)
    Wd = wl.down_weights(2)
    wd8, s_d, _, _ = pack.pack_weights([Wd], None)
    out = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_fp8_split(dev_u8(hid8), dev_u8(wd8), scalar(s_h), scalar(s_d),
                                  [out], [D])
    torch.cuda.synchronize()
    ref = gemm.epilogue(gemm.gemm_exact(hid8, wd8), s_h, s_d)
    assert_gemm_bf16(host_bf16(out), ref, what="down projection 256x2048x8192")
