"""GPU parity of the MXFP4 band: the weight pack (bit-exact: the block
maxima and the power-of-two scaling are exact, the rounding is decided on
the same fp32 values), the AdaRMS producer with MXFP4 output (its y differs
from the oracle's fp64 y by rounding, so a block scale can flip where the
block maximum sits on a power of two and a code where a value sits on a
rounding midpoint: both on at most 0.1 %), and the block-scaled GEMM from
identical MXFP4 operands (fp32 out within 1e-3 of max|ref| of the exact
oracle, bf16 within one ulp more), through the C ABI.
"""

import numpy as np
import pytest
import torch

import norm_quantize_packed_amd as frt
import workloads as wl
from oracle import codecs, ffn, mxfp4, producers, rope
from gpu_util import (Guarded, assert_codes_close, assert_gemm_bf16, assert_gemm_f32, dev_bf16,
                      dev_u8, host_bf16, host_u8, scalar)

pytestmark = pytest.mark.gpu


def _gpu_pack(Ws, bs=None):
    K = Ws[0].shape[1]
    N = sum(w.shape[0] for w in Ws)
    W4 = Guarded(N, K // 2, torch.uint8)
    S4 = Guarded(K // 256, 8 * N, torch.uint8)      # [K/256][N][8]
    bc = torch.empty(N, dtype=torch.bfloat16, device="cuda") if bs is not None else None
    frt.frt_pack_weights_mxfp4([dev_bf16(w) for w in Ws],
                               None if bs is None else [dev_bf16(b) for b in bs],
                               W4.view, S4.view, bc)
    torch.cuda.synchronize()
    W4.check_guards()
    S4.check_guards()
    return (host_u8(W4.view), host_u8(S4.view).reshape(K // 256, N, 8),
            (host_bf16(bc) if bc is not None else None))


def _oracle_pack(Ws):
    W = np.concatenate([codecs.bf16_to_f32(w) for w in Ws], axis=0)
    codes, scales = mxfp4.quantize_mxfp4(W)
    return mxfp4.pack_nibbles(codes), mxfp4.scales_to_gemm_order(scales)


@pytest.mark.parametrize("shapes,K,std", [(((2048, 256, 256)), 2048, 0.02),
                                          (((96, 32)), 512, 1.0),
                                          (((64,)), 4096, 1e-30),
                                          (((40, 24)), 1280, 1.0)])   # K an odd number of 256-runs
def test_pack_bit_exact(shapes, K, std):
    Ws = [wl.random_bf16(900 + i, (n, K), std) for i, n in enumerate(shapes)]
    bs = [wl.random_bf16(950 + i, (n,), 0.02) for i, n in enumerate(shapes)]
    g4, gs, gb = _gpu_pack(Ws, bs)
    r4, rs = _oracle_pack(Ws)
    assert np.array_equal(gs, rs)
    assert np.array_equal(g4, r4)
    assert np.array_equal(gb, np.concatenate(bs))


def _e2m1_ordinal(codes):
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 8, -(c & 7), c & 7)


@pytest.mark.parametrize("M,D", [(256, 2048), (7, 4096), (64, 512), (33, 768)])
def test_ada_norm_mxfp4_vs_oracle(M, D):
    rng = np.random.default_rng(M + D)
    res = wl.random_bf16(1300 + D, (M, D), 1.0)
    x = wl.random_bf16(1301 + D, (M, D), 1.0)
    gate = wl.random_bf16(1302 + D, (D,), 0.1)
    mod = wl.random_bf16(1303 + D, (1, 3 * D), 0.1)
    ref = producers.ada_norm_quant_fp8(res, x, gate, mod, None, 1e-6)
    rc, rs = mxfp4.quantize_mxfp4(ref["y"])
    out4 = Guarded(M, D // 2, torch.uint8)
    sc = Guarded(D // 256, 8 * M, torch.uint8)      # [D/256][M][8]
    rout = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    frt.frt_ada_norm_quant_mxfp4(dev_bf16(res), dev_bf16(mod), out4.view, sc.view, x=dev_bf16(x),
                                 gate=dev_bf16(gate), eps=1e-6, residual_out=rout)
    torch.cuda.synchronize()
    out4.check_guards()
    sc.check_guards()
    assert np.array_equal(host_bf16(rout), ref["residual_out"])
    gs = mxfp4.scales_from_gemm_order(host_u8(sc.view).reshape(D // 256, M, 8))
    gc = mxfp4.unpack_nibbles(host_u8(out4.view))
    same = gs == rs
    assert same.mean() >= 0.999, f"{(~same).sum()} of {same.size} block scales differ"
    bsame = np.repeat(same, 32, axis=1)
    d = np.abs(_e2m1_ordinal(gc) - _e2m1_ordinal(rc))[bsame]
    assert d.max(initial=0) <= 1
    assert (d > 0).mean() <= 0.001, f"{(d > 0).sum()} of {d.size} codes differ"
    del rng


@pytest.mark.parametrize("M,N,K,bias", [
    (1, 6144, 4096, False),     # decode: the small-M plan, rows past M not loaded
    (16, 768, 512, True),
    (64, 2560, 2048, False),
    (256, 2560, 2048, True),    # the decoder layer's QKV (64x64 plan)
    (256, 16384, 2048, False),  # the decoder layer's gate/up (128x128 plan)
    (600, 1024, 1024, False),   # ragged M (64x64 plan)
    (256, 2048, 4096, False),   # 64x32 plan above the small-M band
    # K an odd number of 256-element runs: the 64x32 plans take one run per
    # stage in a deeper ring
    (1, 1024, 768, True),
    (24, 640, 1280, False),
    (40, 512, 1280, False),
    (200, 512, 768, False),
    (256, 2560, 1280, False),   # 64x64 plan
    # N not a multiple of 32: the last 32-row block of B scales is partial
    # (rows past N fetch zeros); one case per plan
    (300, 16300, 512, True),    # 128x128 plan
    (600, 1000, 1024, False),   # 64x64 plan
    (333, 1000, 512, True),     # 64x32 plan
    (5, 1000, 768, False),      # small-M plan
    (3, 1000, 2048, True),      # M <= 8 in one round: five-deep ring
])
def test_gemm_mxfp4_vs_oracle(M, N, K, bias):
    a = wl.random_bf16(1400 + M, (M, K), 1.0)
    ac, as_ = mxfp4.quantize_mxfp4(codecs.bf16_to_f32(a))
    W = wl.random_bf16(1401 + N, (N, K), 0.02)
    w4, ws4, _ = _gpu_pack([W])
    wc = mxfp4.unpack_nibbles(w4)
    wsc = mxfp4.scales_from_gemm_order(ws4)
    b = wl.random_bf16(1402, (N,), 0.02) if bias else None
    splits = [N // 2, N - N // 2]
    outs32 = [torch.empty((M, n), dtype=torch.float32, device="cuda") for n in splits]
    outs16 = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in splits]
    x4, xs = dev_u8(mxfp4.pack_nibbles(ac)), dev_u8(mxfp4.scales_to_gemm_order(as_))
    dw4, dws4 = dev_u8(w4), dev_u8(ws4)
    db = None if b is None else dev_bf16(b)
    frt.frt_packed_gemm_mxfp4_split(x4, xs, dw4, dws4, outs32, splits, db)
    frt.frt_packed_gemm_mxfp4_split(x4, xs, dw4, dws4, outs16, splits, db)
    torch.cuda.synchronize()
    ref = mxfp4.gemm_mxfp4(ac, as_, wc, wsc)
    if b is not None:
        ref = ref + codecs.bf16_to_f32(b).astype(np.float64)[None, :]
    got32 = np.concatenate([o.cpu().numpy() for o in outs32], 1)
    assert_gemm_f32(got32, ref, f"mxfp4 {M}x{N}x{K} fp32")
    got16 = np.concatenate([host_bf16(o) for o in outs16], 1)
    assert_gemm_bf16(got16, ref, f"mxfp4 {M}x{N}x{K} bf16")


@pytest.mark.parametrize("M,K,H,bias", [
    (256, 2048, 8192, False),   # the decoder layer's gate/up (128x128 plan)
    (600, 512, 4000, True),     # 128x128 plan, ragged M and H (last tile half gate columns)
    (600, 1024, 704, False),    # 64x64 plan, ragged M and H
    (40, 1280, 320, True),      # small M; K an odd number of 256-element runs
    (1, 512, 64, False),        # one row, one tile
    (300, 512, 8100, False),    # 128x128 plan, H not a multiple of 32
    (300, 512, 1000, True),     # 64x64 plan, H not a multiple of 32
])
def test_gemm_mxfp4_geglu_vs_unfused_and_oracle(M, K, H, bias):
    """The MXFP4 gate/up GEMM with the GEGLU quantiser as its epilogue: its
    codes equal the split MXFP4 GEMM's bf16 output quantised by the
    standalone GEGLU kernel bit for bit; that bf16 output is within the GEMM
    tolerance of the exact oracle GEMM, and the codes match the oracle's
    GEGLU quantiser on it."""
    a = wl.random_bf16(1500 + M, (M, K), 1.0)
    ac, as_ = mxfp4.quantize_mxfp4(codecs.bf16_to_f32(a))
    Wg = wl.random_bf16(1501 + H, (H, K), 0.02)
    Wu = wl.random_bf16(1502 + H, (H, K), 0.02)
    bs = [wl.random_bf16(1503, (H,), 0.02), wl.random_bf16(1504, (H,), 0.02)] if bias else None
    w4, ws4, bc = _gpu_pack([Wg, Wu], bs)
    x4, xs = dev_u8(mxfp4.pack_nibbles(ac)), dev_u8(mxfp4.scales_to_gemm_order(as_))
    dw4, dws4 = dev_u8(w4), dev_u8(ws4)
    db = None if bc is None else dev_bf16(bc)
    # unfused: bf16 gate|up, then the standalone quantiser
    gu = torch.empty((M, 2 * H), dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_mxfp4_split(x4, xs, dw4, dws4, [gu], [2 * H], db)
    torch.cuda.synchronize()
    gu_bits = host_bf16(gu)
    s_o = producers.calibrate_act_scale(ffn.geglu(gu_bits, H))
    unf = torch.empty((M, H), dtype=torch.uint8, device="cuda")
    frt.frt_geglu_quant_fp8(gu, H, scalar(s_o), out_fp8=unf)
    # fused, into a guarded buffer with a wider row stride
    out = Guarded(M, H, torch.uint8, ld=H + 16)
    frt.frt_packed_gemm_mxfp4_geglu_quant(x4, xs, dw4, dws4, scalar(s_o), out.view, db)
    torch.cuda.synchronize()
    out.check_guards()
    got = host_u8(out.view)
    assert np.array_equal(got, host_u8(unf)), "fused codes differ from the unfused chain"
    ref = mxfp4.gemm_mxfp4(ac, as_, mxfp4.unpack_nibbles(w4), mxfp4.scales_from_gemm_order(ws4))
    if bc is not None:
        ref = ref + codecs.bf16_to_f32(bc).astype(np.float64)[None, :]
    assert_gemm_bf16(gu_bits, ref, f"mxfp4 gate|up {M}x{2 * H}x{K}")
    assert_codes_close(got, ffn.geglu_quant_fp8(gu_bits, H, s_o)["codes"], what=f"mxfp4 geglu {M}x{H}")


def _mx_out(M, W):
    """Guarded code and scale buffers for M rows of W columns."""
    return Guarded(M, W // 2, torch.uint8, ld=W // 2 + 4), Guarded(W // 256, 8 * M, torch.uint8)


def _specials(M, D):
    """bf16 rows with every kind of block: zeros, a NaN, an infinity,
    subnormals, values near the bf16 maximum, exact midpoints of the e2m1
    grid and random values (bit patterns)."""
    x = wl.random_bf16(1600 + D, (M, D), 1.0).copy()
    f = codecs.bf16_to_f32(x)
    if M >= 1:
        f[0, 0:32] = 0.0
        f[0, 32:64] = np.float32(1e-40)        # subnormal block
        f[0, 64:96] *= np.float32(1e37)        # near the top of the range
        # a block whose maximum is 4 (scale 1): 0.25, 0.75, 1.25, ... ties
        f[0, 96:128] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0] * 4, np.float32)
    if M >= 2:
        f[1, 0] = np.nan
        f[1, 40] = np.inf
        f[1, 80] = -np.inf
    return wl.to_bf16_bits(f)


@pytest.mark.parametrize("M,D,pad", [(256, 2048, 0), (7, 4096, 8), (3, 256, 0), (65, 768, 16)])
def test_quantize_mxfp4_bit_exact(M, D, pad):
    """MXFP4 of a bf16 tensor: the scale and every code are decided on the
    exact bf16 values, so both match the oracle bit for bit."""
    x = _specials(M, D)
    xd = torch.zeros((M, D + pad), dtype=torch.bfloat16, device="cuda")
    xd[:, :D] = dev_bf16(x)
    o4, sc = _mx_out(M, D)
    frt.frt_quantize_mxfp4(xd[:, :D], o4.view, sc.view)
    torch.cuda.synchronize()
    o4.check_guards()
    sc.check_guards()
    rc, rs = mxfp4.quantize_mxfp4(codecs.bf16_to_f32(x))
    gs = mxfp4.scales_from_gemm_order(host_u8(sc.view).reshape(D // 256, M, 8))
    assert np.array_equal(gs, rs)
    finite = np.repeat(rs != 255, 32, axis=1)   # codes of a NaN/inf block are unspecified
    assert np.array_equal(mxfp4.unpack_nibbles(host_u8(o4.view))[finite], rc[finite])


@pytest.mark.parametrize("M,H", [(256, 8192), (5, 256), (40, 1280)])
def test_geglu_quant_mxfp4(M, H):
    """GEGLU to MXFP4: the codes and scales equal the oracle's MXFP4 of the
    GPU's own fp32 GEGLU output (the FP8 GEGLU kernel's diagnostic y, formed
    the same way), and against the oracle's fp64 GEGLU the scales agree on
    >= 99.9 % of blocks and the codes within one step on >= 99.9 %."""
    gu = wl.random_bf16(1700 + H, (M, 2 * H), 1.0)
    dgu = dev_bf16(gu)
    o4, sc = _mx_out(M, H)
    frt.frt_geglu_quant_mxfp4(dgu, H, o4.view, sc.view)
    y = torch.empty((M, H), dtype=torch.float32, device="cuda")
    frt.frt_geglu_quant_fp8(dgu, H, None, y_f32=y)
    torch.cuda.synchronize()
    o4.check_guards()
    sc.check_guards()
    gc = mxfp4.unpack_nibbles(host_u8(o4.view))
    gs = mxfp4.scales_from_gemm_order(host_u8(sc.view).reshape(H // 256, M, 8))
    oc, os_ = mxfp4.quantize_mxfp4(y.cpu().numpy())
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)
    rc, rs = mxfp4.quantize_mxfp4(ffn.geglu(gu, H))
    same = gs == rs
    assert same.mean() >= 0.999, f"{(~same).sum()} of {same.size} block scales differ"
    d = np.abs(_e2m1_ordinal(gc) - _e2m1_ordinal(rc))[np.repeat(same, 32, axis=1)]
    assert d.max(initial=0) <= 1
    assert (d > 0).mean() <= 0.001, f"{(d > 0).sum()} of {d.size} codes differ"


_FILL = 0x3C01   # bf16 pattern pre-filled into the caches (rows not written keep it)


def _caches(T, kv, hd):
    k = torch.full((T, kv, hd), _FILL, dtype=torch.int16, device="cuda")
    return k.view(torch.bfloat16), k.clone().view(torch.bfloat16)


@pytest.mark.parametrize("M,K,nh,kv,hd,P,bias", [
    (256, 2048, 8, 1, 256, 768, False),   # the decoder layer's heads (64x64 plan)
    (1024, 512, 32, 8, 128, 0, True),     # 128x128 plan
    (16, 512, 4, 2, 64, 5, True),         # small M: rows past M not loaded
    (8, 2048, 4, 2, 64, 3, False),        # small M, K % 1024 == 0: four-run stages
    (40, 768, 2, 1, 128, 0, False),       # K an odd number of 256-element runs
    (600, 1024, 4, 2, 128, 100, False),   # ragged M
])
def test_gemm_mxfp4_rope_vs_unfused_and_oracle(M, K, nh, kv, hd, P, bias):
    """The MXFP4 QKV GEMM with the split + RoPE + KV-cache epilogue: q and
    the cache rows equal the split MXFP4 GEMM's bf16 output passed through
    the standalone consumer bit for bit; that bf16 output is within the GEMM
    tolerance of the exact oracle, and the consumer on it equals the
    oracle's."""
    a = wl.random_bf16(1800 + M, (M, K), 1.0)
    ac, as_ = mxfp4.quantize_mxfp4(codecs.bf16_to_f32(a))
    Wq = rope.interleave_rows(wl.random_bf16(1801 + hd, (nh * hd, K), 0.02), nh, hd)
    Wk = rope.interleave_rows(wl.random_bf16(1802 + hd, (kv * hd, K), 0.02), kv, hd)
    Wv = wl.random_bf16(1803 + hd, (kv * hd, K), 0.02)
    bs = [wl.random_bf16(1804 + i, (n,), 0.02) for i, n in enumerate((nh * hd, kv * hd, kv * hd))] \
        if bias else None
    w4, ws4, bc = _gpu_pack([Wq, Wk, Wv], bs)
    width = (nh + 2 * kv) * hd
    T = P + M + 3
    table = wl.rope_table(M, hd, P)
    dtab = dev_bf16(table)
    x4, xs = dev_u8(mxfp4.pack_nibbles(ac)), dev_u8(mxfp4.scales_to_gemm_order(as_))
    dw4, dws4 = dev_u8(w4), dev_u8(ws4)
    db = None if bc is None else dev_bf16(bc)
    q = torch.empty((M, nh, hd), dtype=torch.bfloat16, device="cuda")
    kc, vc = _caches(T, kv, hd)
    frt.frt_packed_gemm_mxfp4_qkv_rope(x4, xs, dw4, dws4, nh, kv, hd, dtab, P, q, kc, vc, db)
    qkv = torch.empty((M, width), dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_mxfp4_split(x4, xs, dw4, dws4, [qkv], [width], db)
    q2 = torch.empty_like(q)
    kc2, vc2 = _caches(T, kv, hd)
    frt.frt_qkv_split_rope_kvcache(qkv, dtab, nh, kv, hd, P, q2, kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
    qkv_bits = host_bf16(qkv)
    ref = mxfp4.gemm_mxfp4(ac, as_, mxfp4.unpack_nibbles(w4), mxfp4.scales_from_gemm_order(ws4))
    if bc is not None:
        ref = ref + codecs.bf16_to_f32(bc).astype(np.float64)[None, :]
    assert_gemm_bf16(qkv_bits, ref, f"mxfp4 qkv {M}x{width}x{K}")
    fill = np.full((T, kv, hd), _FILL, np.uint16)
    rq, rk, rv = rope.qkv_split_rope_kvcache(qkv_bits, table, nh, kv, hd, P, fill, fill)
    assert np.array_equal(host_bf16(q).reshape(rq.shape), rq)
    assert np.array_equal(host_bf16(kc), rk)
    assert np.array_equal(host_bf16(vc), rv)


@pytest.mark.parametrize("M,K,H,bias", [
    (256, 2048, 8192, False),   # the decoder layer's gate/up (128x128 plan)
    (600, 1024, 768, True),     # 64x64 plan, ragged M
    (40, 1280, 256, True),      # small M, K an odd number of runs
    (1, 512, 512, False),
])
def test_gemm_mxfp4_geglu_to_mxfp4_vs_unfused(M, K, H, bias):
    """The MXFP4 gate/up GEMM with the GEGLU quantised to MXFP4 in its
    epilogue: codes and scales equal the split MXFP4 GEMM's bf16 output
    passed through the standalone GEGLU -> MXFP4 kernel bit for bit (whose
    agreement with the oracle the GEGLU -> MXFP4 test checks)."""
    a = wl.random_bf16(1900 + M, (M, K), 1.0)
    ac, as_ = mxfp4.quantize_mxfp4(codecs.bf16_to_f32(a))
    Wg = wl.random_bf16(1901 + H, (H, K), 0.02)
    Wu = wl.random_bf16(1902 + H, (H, K), 0.02)
    bs = [wl.random_bf16(1903, (H,), 0.02), wl.random_bf16(1904, (H,), 0.02)] if bias else None
    w4, ws4, bc = _gpu_pack([Wg, Wu], bs)
    x4, xs = dev_u8(mxfp4.pack_nibbles(ac)), dev_u8(mxfp4.scales_to_gemm_order(as_))
    dw4, dws4 = dev_u8(w4), dev_u8(ws4)
    db = None if bc is None else dev_bf16(bc)
    gu = torch.empty((M, 2 * H), dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_mxfp4_split(x4, xs, dw4, dws4, [gu], [2 * H], db)
    u4, us = _mx_out(M, H)
    frt.frt_geglu_quant_mxfp4(gu, H, u4.view, us.view)
    # the epilogue stages its tiles in a ring slot with no block barrier:
    # repeated calls must give the same bytes every time
    for rep in range(3):
        f4, fs = _mx_out(M, H)
        frt.frt_packed_gemm_mxfp4_geglu_mxfp4(x4, xs, dw4, dws4, f4.view, fs.view, db)
        torch.cuda.synchronize()
        for g in (u4, us, f4, fs):
            g.check_guards()
        assert np.array_equal(host_u8(fs.view), host_u8(us.view)), f"block scales differ (call {rep})"
        assert np.array_equal(host_u8(f4.view), host_u8(u4.view)), f"codes differ (call {rep})"
