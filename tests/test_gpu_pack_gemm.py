"""GPU parity of the weight packer (bit-exact) and of the packed FP8 GEMM
(from identical FP8 operands) against the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import norm_quantize_packed_amd as frt
import workloads as wl
from oracle import codecs, gemm, pack
from gpu_util import (Guarded, assert_gemm_bf16, assert_gemm_f32, dev_bf16,
                      dev_u8, host_bf16, host_u8, scalar)

pytestmark = pytest.mark.gpu


def _gpu_pack(Ws, bs, with_bias=True):
    K = Ws[0].shape[1]
    N = sum(w.shape[0] for w in Ws)
    W8 = Guarded(N, K, torch.uint8)
    ws = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    bc = Guarded(1, N, torch.bfloat16) if with_bias else None
    frt.frt_pack_weights_fp8([dev_bf16(w) for w in Ws],
                             None if bs is None else
                             [None if b is None else dev_bf16(b) for b in bs],
                             W8.view, ws, bc.view[0] if bc else None)
    torch.cuda.synchronize()
    W8.check_guards()
    if bc:
        bc.check_guards()
    return (host_u8(W8.view), np.float32(ws.item()),
            host_bf16(bc.view)[0] if bc else None)


@pytest.mark.parametrize("cid,site", [(1, 0), (2, 0), (2, 1), (3, 0), (4, 0)])
def test_pack_workload_bit_exact(cid, site):
    w = wl.weights(cid, site)
    g8, gs, gb = _gpu_pack(w["W"], w["b"])
    r8, rs, rb, _ = pack.pack_weights(w["W"], w["b"])
    assert gs == rs
    assert np.array_equal(gb, rb)
    assert np.array_equal(g8, r8)


def test_pack_full_widest_workload_sampled():
    """Workload 5's 32768 x 16384 gate/up pack: the joint scale exactly, and
    sampled rows bit-exact (the oracle packs those rows under that scale)."""
    w = wl.weights(5, 0)
    g8, gs, _ = _gpu_pack(w["W"], w["b"], with_bias=False)
    amax = max(np.abs(codecs.bf16_to_f32(x)).max() for x in w["W"])
    assert gs == np.float32(max(np.float32(amax / np.float32(448)),
                                np.float32(1e-8)))
    W = np.concatenate(w["W"], axis=0)
    rows = np.random.default_rng(5).integers(0, W.shape[0], 64)
    q = (codecs.bf16_to_f32(W[rows]) / gs).astype(np.float32)
    ref = codecs.e4m3_encode(np.clip(q, -448, 448))
    assert np.array_equal(g8[rows], ref)


def test_pack_every_bf16_pattern_and_odd_shapes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = bits[np.isfinite(codecs.bf16_to_f32(bits))]
    fin = np.concatenate([fin, np.zeros((-fin.size) % 256, np.uint16)])
    W = fin.reshape(-1, 256)
    for Ws in ([W], [W[:100, :255].copy(), W[100:, :255].copy()],
               [(W[:, :200] & np.uint16(0x87FF)).copy()],
               [np.zeros((16, 64), np.uint16)],
               [W[:3, :7].copy(), W[3:9, :7].copy(), W[9:10, :7].copy()]):
        g8, gs, gb = _gpu_pack(Ws, [None] * len(Ws))
        r8, rs, rb, _ = pack.pack_weights(Ws, None)
        assert gs == rs
        assert np.array_equal(g8, r8)
        assert not gb.any()


# ------------------------------------------------------------------ GEMM

def _gpu_gemm(x8, w8, s_a, s_w, bias, splits, *, f32, M=None, ld_pad=0):
    M = x8.shape[0] if M is None else M
    outs = [Guarded(M, n, torch.float32 if f32 else torch.bfloat16,
                    ld=n + ld_pad) for n in splits]
    frt.frt_packed_gemm_fp8_split(
        dev_u8(x8), dev_u8(w8), scalar(s_a), scalar(s_w),
        [o.view for o in outs], splits,
        bias_cat=None if bias is None else dev_bf16(bias), M=M)
    torch.cuda.synchronize()
    for o in outs:
        o.check_guards()
    res = []
    for o in outs:
        if f32:
            res.append(o.view.cpu().numpy())
        else:
            res.append(host_bf16(o.view))
    return res


def _check_gemm(x8, w8, s_a, s_w, bias, splits, what, ld_pad=0):
    ref = gemm.packed_gemm_split(x8, w8, s_a, s_w, bias, splits)
    got32 = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=True, ld_pad=ld_pad)
    got16 = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    scale = max(np.max(np.abs(x)) for x in ref)
    worst = 0.0
    for i, (r, g32, g16) in enumerate(zip(ref, got32, got16)):
        err = np.max(np.abs(g32.astype(np.float64) - r))
        assert err <= 1e-3 * scale, f"{what} split {i}: {err:.3e}"
        worst = max(worst, err / scale)
        assert_gemm_bf16(g16, r, f"{what} split {i}")
    print(f"{what}: fp32 max|d|/max|ref| = {worst:.2e}")
    return ref


def _operands(cid, site, M=None, seed=0):
    if cid == 5:
        # the widest workload's weights are exercised by the pack tests; the
        # GEMM takes random codes of the same shape (identical operands)
        wk = wl.WORKLOADS[5]
        w8 = wl.random_codes(4100, (sum(wk.gemms[0]), wk.D))
        M = wk.rows if M is None else M
        x8 = wl.random_codes(4005 + seed, (M, wk.D))
        return x8, w8, np.float32(0.01), np.float32(0.004), None, list(wk.gemms[0])
    w = wl.weights(cid, site)
    w8, s_w, bias, splits = pack.pack_weights(w["W"], w["b"])
    K = w8.shape[1]
    M = wl.WORKLOADS[cid].rows if M is None else M
    x8 = wl.random_codes(4000 + cid + seed, (M, K))
    # a realistic activation code spread: mostly small magnitudes
    return x8, w8, np.float32(0.01), s_w, (bias if w["b"][0] is not None else None), splits


@pytest.mark.parametrize("cid,site,M", [(1, 0, 16), (2, 0, 256), (2, 1, 256),
                                        (3, 0, 600), (4, 0, 64), (4, 0, 1),
                                        (4, 0, 17), (5, 0, 40),
                                        # tile-plan boundaries: M = 65 leaves
                                        # the small-M plan, 511 is the last
                                        # mid-M size (ragged in M)
                                        (4, 0, 65), (2, 1, 511)])
def test_gemm_workload(cid, site, M):
    x8, w8, s_a, s_w, bias, splits = _operands(cid, site, M)
    _check_gemm(x8, w8, s_a, s_w, bias, splits, f"workload {cid}/{site} M={M}")


@pytest.mark.parametrize("cid", [3, 5])
def test_gemm_full_size_sampled(cid):
    """Full workload size in the bench's launch (bf16 out); sampled outputs
    computed one by one by the oracle."""
    x8, w8, s_a, s_w, bias, splits = _operands(cid, 0)
    M, N = x8.shape[0], w8.shape[0]
    outs = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    full = np.concatenate(outs, axis=1)
    rng = np.random.default_rng(cid)
    rows = np.concatenate([rng.integers(0, M, 2000), [M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, 2000), [N - 1, N - 1]])
    acc = gemm.gemm_exact_at(x8, w8, rows, cols)
    ref = gemm.epilogue(acc, s_a, s_w, None if bias is None else bias[cols])
    # the whole output's scale bounds the accumulation error term
    assert_gemm_bf16(full[rows, cols], ref, f"workload {cid} sampled")


@pytest.mark.parametrize("cid,tp", [(3, 8), (5, 8)])
def test_gemm_tensor_parallel_shard_sampled(cid, tp):
    """One GPU's share of a column-parallel packed GEMM at its real shape
    (rank 0 of 8: 8192 x 3*384 x 3072 with bias, from the workload's own
    weights; 2048 x 2*2048 x 16384 on random codes of that shape): every
    sibling keeps its first N_i / tp rows, and sampled outputs are checked
    one by one against the oracle."""
    wk = wl.WORKLOADS[cid]
    M, K = wk.rows, wk.D
    if cid == 5:
        splits = [n // tp for n in wk.gemms[0]]
        w8 = wl.random_codes(4200 + tp, (sum(splits), K))
        s_w, bias = np.float32(0.004), None
    else:
        ws = wl.tp_shard(wl.weights(cid, 0), tp, 0, wl.TP_UNIT[cid])
        w8, s_w, bias, splits = pack.pack_weights(ws["W"], ws["b"])
    x8 = wl.random_codes(4300 + cid, (M, K))
    s_a = np.float32(0.01)
    outs = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    full = np.concatenate(outs, axis=1)
    N = w8.shape[0]
    rng = np.random.default_rng(cid + tp)
    rows = np.concatenate([rng.integers(0, M, 2000), [M - 1, 0]])
    cols = np.concatenate([rng.integers(0, N, 2000), [N - 1, 0]])
    acc = gemm.gemm_exact_at(x8, w8, rows, cols)
    ref = gemm.epilogue(acc, s_a, s_w, None if bias is None else bias[cols])
    assert_gemm_bf16(full[rows, cols], ref, f"workload {cid} rank 0 of {tp}")


def test_gemm_edges_k_tail_strides_unaligned_splits():
    rng = np.random.default_rng(9)
    for (M, K, splits) in [(33, 528, (100, 28, 200)), (257, 1040, (96, 160)),
                           (5, 4096, (1, 2, 3, 122)), (300, 512, (40,) * 16)]:
        N = sum(splits)
        w8 = wl.random_codes(int(rng.integers(1 << 30)), (N, K))
        x8 = wl.random_codes(int(rng.integers(1 << 30)), (M, K))
        bias = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
        _check_gemm(x8, w8, np.float32(0.003), np.float32(0.002), bias,
                    list(splits), f"M={M} K={K}", ld_pad=6)


@pytest.mark.parametrize("M,K", [(1, 4096), (16, 1024), (17, 1040), (32, 2048),
                                 (65, 1024), (256, 2048)])
def test_gemm_small_tile_epilogue_operands(M, K):
    """The small-tile plans (M = 1 and 16: 16 A rows; 17 and 32: 32 rows;
    65 and 256: the 64x32 split plan) read their epilogue operands ahead of
    the main loop: the scales, each lane's split address and row stride,
    its bias. Sixteen splits whose widths cut the 32-column lane groups
    anywhere, padded row strides, fp32 and bf16 outputs, with a bias and
    without one (the kernel then reads, and ignores, weight bytes in the
    bias's place)."""
    rng = np.random.default_rng(M * 31 + K)
    splits = [37, 5, 64, 1, 90, 33, 31, 128, 7, 9, 100, 3, 44, 20, 11, 29]
    N = sum(splits)
    w8 = wl.random_codes(int(rng.integers(1 << 30)), (N, K))
    x8 = wl.random_codes(int(rng.integers(1 << 30)), (M, K))
    bias = wl.to_bf16_bits(rng.standard_normal(N).astype(np.float32))
    _check_gemm(x8, w8, np.float32(0.003), np.float32(0.002), bias, splits,
                f"M={M} K={K} with bias", ld_pad=6)
    _check_gemm(x8, w8, np.float32(0.003), np.float32(0.002), None, splits,
                f"M={M} K={K} no bias", ld_pad=2)


def test_gemm_joint_slots_share_one_buffer():
    """Two adjacent splits written into one [M, N0 + N1] region through
    offset pointers with a shared row stride (a joint q|k consumer)."""
    x8, w8, s_a, s_w, bias, splits = _operands(1, 0)
    M = x8.shape[0]
    ref = np.concatenate(gemm.packed_gemm_split(x8, w8, s_a, s_w, bias, splits), 1)
    buf = torch.zeros(M, 640, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(M, 128, dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_fp8_split(dev_u8(x8), dev_u8(w8), scalar(s_a),
                                  scalar(s_w), [buf[:, :512], buf[:, 512:], v],
                                  splits, bias_cat=None)
    torch.cuda.synchronize()
    got = np.concatenate([host_bf16(buf), host_bf16(v)], 1)
    assert_gemm_bf16(got, ref, "joint slots")


def test_gemm_row_capacity_writes_only_m_rows():
    x8, w8, s_a, s_w, bias, splits = _operands(4, 0, 64)
    out = [torch.full((64, n), 1.5, dtype=torch.bfloat16, device="cuda")
           for n in splits]
    frt.frt_packed_gemm_fp8_split(dev_u8(x8), dev_u8(w8), scalar(s_a),
                                  scalar(s_w), out, splits, M=10)
    torch.cuda.synchronize()
    for o in out:
        assert (o[10:].float() == 1.5).all()


def test_gemm_repeatable_across_calls_and_shapes():
    """Small-M shapes of different tile plans, called repeatedly and
    interleaved: results match the oracle and are bit-identical across
    calls (no state carried from one call or shape to the next)."""
    shapes = [(64, 6144, 4096), (1, 6144, 4096), (16, 768, 512), (40, 2048, 1152)]
    first = {}
    for rep in range(3):
        for (M, N, K) in shapes:
            x8 = wl.random_codes(M * 7 + K, (M, K))
            w8 = wl.random_codes(N * 3 + K, (N, K))
            splits = [N // 2, N - N // 2]
            got = _gpu_gemm(x8, w8, np.float32(0.01), np.float32(0.002), None,
                            splits, f32=True)
            out = np.concatenate(got, 1)
            if rep == 0:
                ref = np.concatenate(gemm.packed_gemm_split(
                    x8, w8, np.float32(0.01), np.float32(0.002), None, splits), 1)
                assert_gemm_f32(out, ref, f"{M}x{N}x{K}")
                first[(M, N, K)] = out
            else:
                assert np.array_equal(out, first[(M, N, K)]), f"{M}x{N}x{K} rep {rep}"


@pytest.mark.parametrize("K", [1024, 1040])
def test_gemm_large_full_grid(K):
    """Large-M plan at a shape with a partial last round (4096 x 6144: 384
    tiles of 256 x 256 on 256 CUs). Every output is checked (fp32 out), with
    a ragged K, and repeated calls are bit-identical."""
    M, N = 4096, 6144
    x8 = wl.random_codes(777 + K, (M, K))
    w8 = wl.random_codes(778 + K, (N, K))
    splits = [4096, 2048]
    ref = np.concatenate(gemm.packed_gemm_split(
        x8, w8, np.float32(0.01), np.float32(0.002), None, splits), 1)
    first = None
    for rep in range(2):
        out = np.concatenate(_gpu_gemm(x8, w8, np.float32(0.01), np.float32(0.002),
                                       None, splits, f32=True), 1)
        if first is None:
            assert_gemm_f32(out, ref, f"{M}x{N}x{K}")
            first = out
        else:
            assert np.array_equal(out, first), f"{M}x{N}x{K} rep {rep}"


def test_gemm_large_vector_stores_match_per_element_stores():
    """The 256x256 plan (2000 x 5000 x 528 takes it: 160 tiles, one round)
    stores bf16 results 16 bytes a lane when every split width and row
    stride is a multiple of 8 elements; a padded stride (ld = n + 6) takes
    the per-element stores. Ragged M, N and K, a bias, and a split boundary
    inside a tile: both give the same bits, match the oracle, and write
    nothing outside their outputs."""
    rng = np.random.default_rng(31)
    M, K, splits = 2000, 528, [3000, 2000]
    N = sum(splits)
    x8 = wl.random_codes(5101, (M, K))
    w8 = wl.random_codes(5102, (N, K))
    bias = wl.to_bf16_bits(0.05 * rng.standard_normal(N).astype(np.float32))
    s_a, s_w = np.float32(0.003), np.float32(0.002)
    ref = gemm.packed_gemm_split(x8, w8, s_a, s_w, bias, splits)
    vec = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    lane = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False, ld_pad=6)
    for i, (a, b, r) in enumerate(zip(vec, lane, ref)):
        assert np.array_equal(a, b), f"split {i}: vector and per-element stores differ"
        assert_gemm_bf16(a, r, f"2000x5000x528 split {i}")


@pytest.mark.parametrize("K", [2048, 3088, 6160])
@pytest.mark.parametrize("splits", [[5000, 2400, 1600], [4000, 2400, 1600]])
def test_gemm_deep_k_plan_full_grid(K, splits):
    """The four-wave 256-row plans (five-unit ring) at deeper K: 2000 x 9000
    takes 256 x 192 tiles (376 tiles against 288 of 256 x 256: two rounds
    either way), 2000 x 8000 takes 256 x 256 tiles (256 tiles, one round;
    256 x 192 would need two); ragged M and N, a
    bias, three splits whose boundaries fall inside tiles and, at K = 3088
    and 6160, a K tail. Every fp32 output is checked against the oracle; the
    16-byte bf16 stores and the per-element stores of a padded stride give
    the same bits, match the oracle and write nothing outside their outputs;
    a second call repeats the bits."""
    rng = np.random.default_rng(K)
    M = 2000
    N = sum(splits)
    x8 = wl.random_codes(6101 + K, (M, K))
    w8 = wl.random_codes(6102 + K + N, (N, K))
    bias = wl.to_bf16_bits(0.05 * rng.standard_normal(N).astype(np.float32))
    s_a, s_w = np.float32(0.003), np.float32(0.002)
    ref = gemm.packed_gemm_split(x8, w8, s_a, s_w, bias, splits)
    f32 = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=True)
    for i, (g, r) in enumerate(zip(f32, ref)):
        assert_gemm_f32(g, r, f"2000x{N}x{K} fp32 split {i}")
    vec = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    lane = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False, ld_pad=6)
    again = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    for i, (a, b, c, r) in enumerate(zip(vec, lane, again, ref)):
        assert np.array_equal(a, b), f"split {i}: vector and per-element stores differ"
        assert np.array_equal(a, c), f"split {i}: repeated call differs"
        assert_gemm_bf16(a, r, f"2000x{N}x{K} split {i}")


def test_gemm_256_plan_with_a_narrow_tail_launch():
    """4000 x 17000 on the 256-row plan: 16 x 67 tiles of 256 x 256 would
    leave a partial fifth round, so the columns below 16384 run as 1024
    tiles of 256 x 256 (four whole rounds) and the last 616 columns as a
    second launch of 256 x 128 tiles. Ragged M, N and K, a bias, splits whose
    boundaries fall on both sides of the seam: every fp32 output matches the
    oracle; 16-byte and per-element bf16 stores give the same bits."""
    rng = np.random.default_rng(17)
    M, K, splits = 4000, 1040, [9000, 5000, 3000]
    N = sum(splits)
    x8 = wl.random_codes(7101, (M, K))
    w8 = wl.random_codes(7102, (N, K))
    bias = wl.to_bf16_bits(0.05 * rng.standard_normal(N).astype(np.float32))
    s_a, s_w = np.float32(0.003), np.float32(0.002)
    ref = gemm.packed_gemm_split(x8, w8, s_a, s_w, bias, splits)
    f32 = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=True)
    for i, (g, r) in enumerate(zip(f32, ref)):
        assert_gemm_f32(g, r, f"4000x17000x1040 fp32 split {i}")
    vec = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False)
    lane = _gpu_gemm(x8, w8, s_a, s_w, bias, splits, f32=False, ld_pad=6)
    for i, (a, b, r) in enumerate(zip(vec, lane, ref)):
        assert np.array_equal(a, b), f"split {i}: vector and per-element stores differ"
        assert_gemm_bf16(a, r, f"4000x17000x1040 split {i}")


def test_gemm_deep_k_plan_row_capacity():
    """M below the buffers' rows on the deep-K 256x256 plan (the last row of
    tiles is partial): rows past M are neither written nor read."""
    M, K, N = 1900, 6144, 5120
    x8 = wl.random_codes(6301, (2048, K))
    w8 = wl.random_codes(6302, (N, K))
    out = torch.full((2048, N), 1.5, dtype=torch.bfloat16, device="cuda")
    frt.frt_packed_gemm_fp8_split(dev_u8(x8), dev_u8(w8), scalar(0.01), scalar(0.002),
                                  [out], [N], M=M)
    torch.cuda.synchronize()
    assert (out[M:].float() == 1.5).all()
    ref = gemm.packed_gemm_split(x8[:M], w8, np.float32(0.01), np.float32(0.002), None, [N])[0]
    assert_gemm_bf16(host_bf16(out[:M]), ref, "deep-K M=1900")
