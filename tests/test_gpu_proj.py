"""GPU parity of the projections without a producer: the static FP8
quantiser of a bf16 tensor (the O projection's input) and the bf16-input
packed GEMM, against the oracle through the C ABI.

The quantiser's input is exact in fp32 and its division correctly rounded,
so its codes must equal the oracle's bit for bit. The bf16-input GEMM must
write exactly those codes into its FP8 buffer and then produce what the FP8
GEMM produces on them (bit for bit), which is within the GEMM tolerance of
the exact oracle.
"""

import numpy as np
import pytest
import torch

import norm_quantize_packed_amd as frt
import workloads as wl
from oracle import codecs, gemm, pack, producers
from gpu_util import (Guarded, assert_gemm_bf16, dev_bf16, dev_u8, host_bf16,
                      host_u8, scalar)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,D,extra", [(256, 2048, 0), (7, 1024, 8), (5, 1001, 3), (1, 8, 0)])
def test_quantize_bit_exact(M, D, extra):
    x = wl.random_bf16(300 + D, (M, D + extra), 3.0)
    xf = codecs.bf16_to_f32(x[:, :D]).astype(np.float64)
    s = producers.calibrate_act_scale(xf)
    ref = producers.quantize_static(xf, s)
    out = Guarded(M, D, torch.uint8, ld=D + (extra // 2) * 2)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    dx = dev_bf16(x)
    frt.frt_quantize_fp8_static(dx[:, :D], scalar(s), out_fp8=out.view, amax_out=amax)
    torch.cuda.synchronize()
    out.check_guards()
    assert np.array_equal(host_u8(out.view), ref)
    assert amax.item() == np.float32(np.max(np.abs(xf)))


def test_quantize_saturates_and_signs():
    v = np.array([[1e5, -1e5, 0.0, -0.0, 1e-30, -1e-30, 448.0, -464.0]], np.float32)
    x = wl.to_bf16_bits(v)
    out = torch.empty((1, 8), dtype=torch.uint8, device="cuda")
    frt.frt_quantize_fp8_static(dev_bf16(x), scalar(1.0), out_fp8=out)
    torch.cuda.synchronize()
    ref = producers.quantize_static(codecs.bf16_to_f32(x).astype(np.float64), np.float32(1.0))
    assert np.array_equal(host_u8(out), ref)
    assert host_u8(out)[0, :2].tolist() == [0x7E, 0xFE]


@pytest.mark.parametrize("M,K,splits,bias", [
    (256, 2048, (2048,), False),       # the decoder layer's O projection
    (16, 1024, (512, 256, 256), True),
    (600, 1040, (300, 212), True),     # K tail, ragged M
])
def test_gemm_bf16in_vs_oracle(M, K, splits, bias):
    x = wl.random_bf16(400 + M, (M, K), 1.0)
    xf = codecs.bf16_to_f32(x).astype(np.float64)
    s_a = producers.calibrate_act_scale(xf)
    codes = producers.quantize_static(xf, s_a)
    Ws = [wl.random_bf16(410 + i, (n, K), 0.02) for i, n in enumerate(splits)]
    bs = [wl.random_bf16(420 + i, (n,), 0.02) for i, n in enumerate(splits)] if bias else None
    w8, s_w, bias_cat, _ = pack.pack_weights(Ws, bs)
    bc = dev_bf16(bias_cat) if bias else None
    x8 = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in splits]
    frt.frt_packed_gemm_bf16in_split(dev_bf16(x), x8, dev_u8(w8), scalar(s_a), scalar(s_w), outs,
                                     list(splits), bc)
    ref_outs = [torch.empty_like(o) for o in outs]
    frt.frt_packed_gemm_fp8_split(dev_u8(codes), dev_u8(w8), scalar(s_a), scalar(s_w), ref_outs,
                                  list(splits), bc)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(x8), codes)
    for o, r in zip(outs, ref_outs):
        assert torch.equal(o.view(torch.int16), r.view(torch.int16))
    exact = gemm.packed_gemm_split(codes, w8, s_a, s_w, bias_cat if bias else None, list(splits))
    for i, (o, e) in enumerate(zip(outs, exact)):
        assert_gemm_bf16(host_bf16(o), e, what=f"bf16-in split {i}")
