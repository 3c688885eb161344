"""GPU parity of the attention-head consumer of the QKV GEMM: the pack-time
pair interleave, the QKV split + adjacent-pair RoPE + KV-cache write
(standalone), and the QKV GEMM with that consumer as its epilogue, against
the oracle through the C ABI.

The rotation is exact before its single bf16 rounding (both products of two
bf16 values are exact in fp32), so q and the cache rows must match the
oracle bit for bit when both start from the same bf16 QKV values. The fused
GEMM is checked in three links: its outputs equal the unfused chain's on
the GPU (split GEMM, bf16 out, then the standalone consumer) bit for bit;
that bf16 QKV output is within the GEMM tolerance of the exact oracle GEMM;
the consumer on it equals the oracle's.
"""

import numpy as np
import pytest
import torch

import norm_quantize_packed_amd as frt
import workloads as wl
from oracle import codecs, gemm, pack, producers, rope
from gpu_util import assert_gemm_bf16, dev_bf16, dev_u8, host_bf16, scalar

pytestmark = pytest.mark.gpu

FILL = 0x3C01   # bf16 pattern pre-filled into the caches (rows not written keep it)


@pytest.mark.parametrize("nheads,hd,K", [(8, 256, 2048), (1, 256, 2048), (3, 6, 100)])
def test_interleave_bit_exact(nheads, hd, K):
    w = wl.random_bf16(11 + K, (nheads * hd, K))
    out = torch.full((nheads * hd, K), 0, dtype=torch.bfloat16, device="cuda")
    frt.frt_interleave_pairs_bf16(dev_bf16(w), out, nheads, hd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(out), rope.interleave_rows(w, nheads, hd))


def _caches(T, kv, hd):
    k = torch.full((T, kv, hd), 0, dtype=torch.int16, device="cuda")
    k.fill_(FILL)
    v = k.clone()
    return k.view(torch.bfloat16), v.view(torch.bfloat16)


def _check_outputs(q, kc, vc, qkv_bits, table, nh, kv, hd, P, what):
    T = kc.shape[0]
    fill = np.full((T, kv, hd), FILL, np.uint16)
    rq, rk, rv = rope.qkv_split_rope_kvcache(qkv_bits, table, nh, kv, hd, P, fill, fill)
    assert np.array_equal(host_bf16(q).reshape(rq.shape), rq), f"{what}: q"
    assert np.array_equal(host_bf16(kc), rk), f"{what}: k cache"
    assert np.array_equal(host_bf16(vc), rv), f"{what}: v cache"


@pytest.mark.parametrize("S,nh,kv,hd,P,T,extra", [
    (256, 8, 1, 256, 768, 1024, 0),   # the decoder layer's heads (vector path)
    (5, 3, 2, 64, 2, 9, 8),           # wider qkv row stride, two KV heads
    (3, 2, 1, 6, 0, 3, 2),            # hd % 8 != 0: the pair-per-thread path
    (1, 1, 1, 2, 0, 1, 0),            # one token, one pair per head
])
def test_rope_split_vs_oracle(S, nh, kv, hd, P, T, extra):
    width = (nh + 2 * kv) * hd
    qkv = wl.random_bf16(200 + hd, (S, width + extra))
    table = wl.rope_table(S, hd, P)
    q = torch.empty((S, nh, hd), dtype=torch.bfloat16, device="cuda")
    kc, vc = _caches(T, kv, hd)
    d = dev_bf16(qkv)
    frt.frt_qkv_split_rope_kvcache(d, dev_bf16(table), nh, kv, hd, P, q, kc, vc)
    torch.cuda.synchronize()
    _check_outputs(q, kc, vc, qkv[:, :width], table, nh, kv, hd, P, f"split S={S} hd={hd}")


def _qkv_operands(M, K, nh, kv, hd, seed, bias=False):
    """FP8 activations and the packed [q; k; v] weight with q and k
    pair-interleaved (oracle permutation and packer)."""
    x = wl.random_bf16(seed, (M, K), 1.0)
    xf = codecs.bf16_to_f32(x).astype(np.float64)
    s_a = producers.calibrate_act_scale(xf)
    x8 = producers.quantize_static(xf, s_a)
    Wq = rope.interleave_rows(wl.random_bf16(seed + 1, (nh * hd, K), 0.02), nh, hd)
    Wk = rope.interleave_rows(wl.random_bf16(seed + 2, (kv * hd, K), 0.02), kv, hd)
    Wv = wl.random_bf16(seed + 3, (kv * hd, K), 0.02)
    bs = [wl.random_bf16(seed + 4 + i, (n,), 0.02) for i, n in enumerate((nh * hd, kv * hd, kv * hd))] \
        if bias else None
    w8, s_w, bias_cat, _ = pack.pack_weights([Wq, Wk, Wv], bs)
    return x8, s_a, w8, s_w, (bias_cat if bias else None)


@pytest.mark.parametrize("M,K,nh,kv,hd,P,bias", [
    (256, 2048, 8, 1, 256, 768, False),   # decoder layer (64x64 plan)
    (16, 2048, 8, 1, 256, 0, True),       # small M, rows past M not loaded
    (3, 2048, 8, 1, 256, 11, True),       # M <= 8 in one round: five-deep ring
    (1, 4096, 32, 8, 128, 0, False),      # one decode token, 6144 x 4096
    (40, 1040, 4, 2, 64, 5, False),       # K tail, two KV heads
    (600, 1024, 4, 2, 128, 100, False),   # ragged M > 512 (64x64 plan)
    (256, 512, 32, 8, 128, 7, False),     # 64x64 plan (ties with 128x128)
    (1024, 512, 32, 8, 128, 0, True),     # 128x128 plan (ties with 256x256)
    (2048, 512, 32, 8, 128, 3, False),    # 256x256 plan
    (2000, 6144, 32, 8, 128, 9, True),    # deep-K 256x256 plan, ragged M, bias
    (2000, 2048, 32, 8, 128, 5, False),   # deep-K plan at its K threshold
])
def test_gemm_rope_vs_oracle_and_unfused(M, K, nh, kv, hd, P, bias):
    x8, s_a, w8, s_w, bc = _qkv_operands(M, K, nh, kv, hd, 700 + M, bias)
    width = (nh + 2 * kv) * hd
    T = P + M + 3
    table = wl.rope_table(M, hd, P)
    dtab = dev_bf16(table)
    # fused
    q = torch.empty((M, nh, hd), dtype=torch.bfloat16, device="cuda")
    kc, vc = _caches(T, kv, hd)
    frt.frt_packed_gemm_fp8_qkv_rope(dev_u8(x8), dev_u8(w8), scalar(s_a), scalar(s_w), nh, kv, hd,
                                     dtab, P, q, kc, vc, None if bc is None else dev_bf16(bc))
    # unfused: bf16 QKV, then the standalone consumer
    qkv = torch.empty((M, width), dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_fp8_split(dev_u8(x8), dev_u8(w8), scalar(s_a), scalar(s_w), [qkv], [width],
                                  None if bc is None else dev_bf16(bc))
    q2 = torch.empty_like(q)
    kc2, vc2 = _caches(T, kv, hd)
    frt.frt_qkv_split_rope_kvcache(qkv, dtab, nh, kv, hd, P, q2, kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
    qkv_bits = host_bf16(qkv)
    exact = gemm.epilogue(gemm.gemm_exact(x8, w8), s_a, s_w, bc)
    assert_gemm_bf16(qkv_bits, exact, what=f"qkv {M}x{width}x{K}")
    _check_outputs(q, kc, vc, qkv_bits, table, nh, kv, hd, P, f"fused M={M}")
