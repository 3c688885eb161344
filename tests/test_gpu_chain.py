"""End to end on the GPU: producer -> packed GEMM, both in HIP, against the
oracle's producer -> oracle GEMM on the same seeded inputs.

The GPU's codes may differ from the oracle's by one e4m3 step on at most
0.1 % of the elements (exact ties); the GEMM output is therefore compared
with the spec GEMM tolerance, 1e-3 * max|ref|, on fp32 outputs."""

import numpy as np
import pytest
import torch

import norm_quantize_packed_amd as frt
import workloads as wl
from oracle import gemm, pack, producers
from gpu_util import assert_gemm_f32, dev_bf16, dev_f32, scalar

pytestmark = pytest.mark.gpu
EPS = wl.EPS


def _packed_gpu(w):
    K = w["W"][0].shape[1]
    N = sum(x.shape[0] for x in w["W"])
    W8 = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    ws = torch.empty(1, dtype=torch.float32, device="cuda")
    bc = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    frt.frt_pack_weights_fp8([dev_bf16(x) for x in w["W"]],
                             [None if b is None else dev_bf16(b) for b in w["b"]],
                             W8, ws, bc)
    return W8, ws, bc


@pytest.mark.parametrize("cid", [1, 4])
def test_chain_adarms(cid):
    cal = wl.producer_inputs(cid, calib=True)
    s = producers.calibrate_act_scale(producers.ada_norm_quant_fp8(
        cal["residual"], cal["x"], cal["gate"], cal["mod"], None, EPS)["y"])
    inp = wl.producer_inputs(cid)
    w = wl.weights(cid, 0)
    r = producers.ada_norm_quant_fp8(inp["residual"], inp["x"], inp["gate"],
                                     inp["mod"], s, EPS)
    w8, s_w, bias, splits = pack.pack_weights(w["W"], w["b"])
    ref = np.concatenate(gemm.packed_gemm_split(r["codes"], w8, s, s_w,
                                                None, splits), 1)
    M, D = inp["rows"], inp["D"]
    x8 = torch.empty(M, D, dtype=torch.uint8, device="cuda")
    frt.frt_ada_norm_quant_fp8(dev_bf16(inp["residual"]), dev_bf16(inp["mod"]),
                               scalar(s), x=dev_bf16(inp["x"]),
                               gate=dev_bf16(inp["gate"]), eps=EPS,
                               out_fp8=x8)
    W8, ws, _ = _packed_gpu(w)
    outs = [torch.empty(M, n, dtype=torch.float32, device="cuda") for n in splits]
    frt.frt_packed_gemm_fp8_split(x8, W8, scalar(s), ws, outs, splits)
    torch.cuda.synchronize()
    got = np.concatenate([o.cpu().numpy() for o in outs], 1)
    assert_gemm_f32(got, ref, f"chain {cid}")


def test_chain_ptok_workload3_slice():
    rows = 300
    cal = wl.producer_inputs(3, calib=True, rows=rows)
    c = producers.ptok_norm_quant_fp8(cal["x"], cal["temb"], cal["table"], None,
                                      0, 1, EPS)
    s = producers.calibrate_act_scale(c["y"])
    inp = wl.producer_inputs(3, rows=rows)
    r = producers.ptok_norm_quant_fp8(inp["x"], inp["temb"], inp["table"], s,
                                      0, 1, EPS)
    w = wl.weights(3, 0)
    w8, s_w, bias, splits = pack.pack_weights(w["W"], w["b"])
    ref = np.concatenate(gemm.packed_gemm_split(r["codes"], w8, s, s_w, bias,
                                                splits), 1)
    x8 = torch.empty(rows, 3072, dtype=torch.uint8, device="cuda")
    frt.frt_ptok_table_norm_quant_fp8(dev_bf16(inp["x"]),
                                      dev_bf16(inp["temb"].reshape(rows, -1)),
                                      dev_f32(inp["table"]), scalar(s), 0, 1,
                                      eps=EPS, out_fp8=x8)
    W8, ws, bc = _packed_gpu(w)
    outs = [torch.empty(rows, n, dtype=torch.float32, device="cuda") for n in splits]
    frt.frt_packed_gemm_fp8_split(x8, W8, scalar(s), ws, outs, splits, bias_cat=bc)
    torch.cuda.synchronize()
    got = np.concatenate([o.cpu().numpy() for o in outs], 1)
    assert_gemm_f32(got, ref, "chain 3")
