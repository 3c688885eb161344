"""Pins for the oracle's weight packer and packed GEMM (CPU only).

The packer is pinned to torch CPU executing the pages' own packing
expression (torch's amax, division and float8_e4m3fn cast are independent of
the oracle's codecs), to invariants of the joint scale, and to closed forms.
The GEMM is pinned to a brute-force triple loop in exact rational arithmetic,
to one-hot closed forms, and to the sibling-concatenation invariant.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, gemm, pack
import workloads as wl
from workloads import random_codes, to_bf16_bits


def _bf(a):
    return to_bf16_bits(np.asarray(a, np.float32))


def _torch_pack(Ws, bs):
    """The pages' packing expression (impls/qkv_pack/fp8_static.py,
    _pack_weights), run by torch on the CPU."""
    ws = [torch.from_numpy(w.view(np.int16)).view(torch.bfloat16) for w in Ws]
    w = torch.cat(ws, 0)
    scale = (w.float().abs().max() / 448.0).clamp(min=1e-8).view(1)
    w8 = (w.float() / scale).clamp(-448, 448).to(torch.float8_e4m3fn)
    biases = []
    for wi, b in zip(ws, bs):
        biases.append(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
                      if b is not None else
                      torch.zeros(wi.shape[0], dtype=torch.bfloat16))
    return (w8.view(torch.uint8).numpy(), scale.numpy()[0],
            torch.cat(biases).view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("std", [0.02, 1.0, 1e-30])
def test_pack_matches_pages_expression_in_torch(std):
    rng = np.random.default_rng(20)
    Ws = [_bf(rng.standard_normal((n, 256)) * std) for n in (96, 32, 32)]
    bs = [_bf(rng.standard_normal(96) * 0.02), None,
          _bf(rng.standard_normal(32))]
    w8, s, bias, splits = pack.pack_weights(Ws, bs)
    t8, ts, tb = _torch_pack(Ws, bs)
    assert np.array_equal(w8, t8)
    assert s == ts
    assert np.array_equal(bias, tb)
    assert splits == [96, 32, 32]


def test_pack_every_bf16_pattern():
    """All finite bf16 bit patterns as weights against torch's cast."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_to_f32(bits)
    bits = bits[np.isfinite(f)]
    bits = np.concatenate([bits, np.zeros((-bits.size) % 256, np.uint16)])
    W = bits.reshape(-1, 256)
    for Wsub in (W, W[:, :128] & np.uint16(0x87FF)):   # wide and narrow amax
        w8, s, _, _ = pack.pack_weights([Wsub])
        t8, ts, _ = _torch_pack([Wsub], [None])
        assert s == ts and np.array_equal(w8, t8)


def test_pack_joint_scale_is_max_of_sibling_scales():
    rng = np.random.default_rng(21)
    Ws = [_bf(rng.standard_normal((64, 128)) * s) for s in (0.5, 2.0, 0.1)]
    _, s, _, _ = pack.pack_weights(Ws)
    per = [pack.pack_weights([w])[1] for w in Ws]
    assert s == max(per)


def test_pack_extremes_and_zero():
    rng = np.random.default_rng(22)
    W = _bf(rng.standard_normal((32, 128)))
    w8, s, _, _ = pack.pack_weights([W])
    Wf = codecs.bf16_to_f32(W)
    i = np.unravel_index(np.argmax(np.abs(Wf)), Wf.shape)
    assert w8[i] & 0x7F == 0x7E            # the amax element maps to 448
    assert np.abs(codecs.e4m3_ordinal(w8)).max() == 126
    z8, zs, zb, _ = pack.pack_weights([np.zeros((16, 64), np.uint16)])
    assert zs == np.float32(1e-8) and not z8.any() and not zb.any()


def test_pack_representable_multiples_are_exact():
    """Weights that are exact multiples s * v of e4m3 values v (with the
    amax fixed at 448 s) decode back to themselves."""
    s = np.float32(2.0 ** -6)     # amax = 7: s = fl32(7/448) = 2^-6 exactly
    vals = np.array([448, -448, 1, -1.125, 0.25, 2 ** -9, 3.5, 0], np.float64)
    W = _bf((vals * float(s))[None, :].astype(np.float32))
    w8, s_got, _, _ = pack.pack_weights([W])
    assert s_got == s
    assert np.array_equal(codecs.e4m3_decode(w8)[0], vals)


def _brute_gemm(x8, w8):
    dec = lambda c: Fraction(int(codecs.e4m3_int(np.uint8([c]))[0]), 512)
    M, K = x8.shape
    N = w8.shape[0]
    out = np.empty((M, N), object)
    for m in range(M):
        for n in range(N):
            out[m, n] = sum(dec(x8[m, k]) * dec(w8[n, k]) for k in range(K))
    return out


def test_gemm_brute_force_tiny_nonsquare():
    x8 = random_codes(30, (3, 40))
    w8 = random_codes(31, (5, 40))
    ref = _brute_gemm(x8, w8)
    got = gemm.gemm_exact(x8, w8)
    for m in range(3):
        for n in range(5):
            assert Fraction(got[m, n]) == ref[m, n]
    # transposed operands must not agree (guards an operand swap)
    assert gemm.gemm_exact(w8[:3], x8).shape == (3, 3)


def test_gemm_one_hot_rows():
    K, N = 64, 24
    w8 = random_codes(32, (N, K))
    x8 = np.zeros((K, K), np.uint8)
    x8[np.arange(K), np.arange(K)] = 0x38           # 1.0 on the diagonal
    acc = gemm.gemm_exact(x8, w8)
    assert np.array_equal(acc, codecs.e4m3_decode(w8).T)
    out = gemm.epilogue(acc, np.float32(0.5), np.float32(0.25))
    assert np.array_equal(out, 0.125 * codecs.e4m3_decode(w8).T)


def test_gemm_exact_at_extremes_long_k():
    """K = 16384 products of the largest code: exact, no overflow."""
    K = 16384
    x8 = np.full((2, K), 0x7E, np.uint8)
    x8[1] = 0xFE
    w8 = np.full((3, K), 0x7E, np.uint8)
    acc = gemm.gemm_exact(x8, w8)
    assert acc[0, 0] == K * 448.0 * 448.0 and acc[1, 2] == -K * 448.0 * 448.0
    at = gemm.gemm_exact_at(x8, w8, np.array([0, 1]), np.array([1, 2]))
    assert np.array_equal(at, [acc[0, 1], acc[1, 2]])


def test_gemm_sampled_matches_full():
    x8 = random_codes(33, (17, 640))
    w8 = random_codes(34, (70, 640))
    acc = gemm.gemm_exact(x8, w8)
    rng = np.random.default_rng(35)
    rows, cols = rng.integers(0, 17, 300), rng.integers(0, 70, 300)
    assert np.array_equal(gemm.gemm_exact_at(x8, w8, rows, cols),
                          acc[rows, cols])


def test_packed_equals_concatenated_sibling_gemms():
    rng = np.random.default_rng(36)
    K = 256
    Ws = [_bf(rng.standard_normal((n, K)) * 0.02) for n in (64, 16, 16)]
    bs = [_bf(rng.standard_normal(n) * 0.02) for n in (64, 16, 16)]
    w8, s, bias, splits = pack.pack_weights(Ws, bs)
    x8 = random_codes(37, (9, K))
    outs = gemm.packed_gemm_split(x8, w8, np.float32(0.01), s, bias, splits)
    off = 0
    for i, n in enumerate(splits):
        sib = gemm.epilogue(gemm.gemm_exact(x8, w8[off:off + n]),
                            np.float32(0.01), s, bs[i])
        assert np.array_equal(outs[i], sib)
        off += n


def test_epilogue_alpha_and_bias():
    acc = np.array([[1.0, -2.0]])
    b = _bf(np.array([0.5, 0.25], np.float32))
    out = gemm.epilogue(acc, np.float32(3.0), np.float32(0.5), b)
    assert np.array_equal(out, [[2.0, -2.75]])
    assert gemm.to_bf16_ref(out)[0, 0] == 0x4000


def test_column_parallel_shards_keep_the_joint_scale():
    """Column-parallel sharding of a packed GEMM (each rank keeps N_i / tp
    rows of every sibling): the maximum of the ranks' own scales, which a
    4-byte all-reduce(MAX) at bind gives, is the single-GPU joint scale
    (amax / 448 and the 1e-8 floor are monotone in amax), and a rank whose
    slice holds the global maximum packs exactly its rows of the
    single-GPU pack."""
    ws = wl.weights(1, 0)
    tp = 2
    w8, s, _, splits = pack.pack_weights(ws["W"], ws["b"])
    shards = [wl.tp_shard(ws, tp, r, 64) for r in range(tp)]
    local = [pack.pack_weights(sh["W"], sh["b"]) for sh in shards]
    assert [list(sh["splits"]) for sh in shards] == [[n // tp for n in splits]] * tp
    assert max(lp[1] for lp in local) == s
    r = int(np.argmax([lp[1] for lp in local]))
    offs = np.cumsum([0] + list(splits))
    rows = np.concatenate([np.arange(o + r * n // tp, o + (r + 1) * n // tp)
                           for o, n in zip(offs[:-1], splits)])
    assert np.array_equal(local[r][0], w8[rows])
    with pytest.raises(ValueError):
        wl.tp_shard(ws, 3, 0, 64)
