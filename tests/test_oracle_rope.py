"""Pins for the oracle's QKV split + adjacent-pair RoPE + KV-cache write
(CPU only).

The central pin is the equivalence the pages establish at bind: rotating
adjacent pairs on the pack-permuted layout equals the host's rotate-half
RoPE (``x * cos + rotate_half(x) * sin``, written here with torch from its
usual definition) followed by the same permutation. Further pins: the
permutation itself on a small head, special angles, angle composition,
norm preservation, and the split / cache placement on a brute-force loop.
"""

import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import codecs, rope


def _bf(a):
    return wl.to_bf16_bits(np.asarray(a, np.float32))


def test_pair_perm_small_head():
    assert rope.pair_perm(4).tolist() == [0, 2, 1, 3]
    assert rope.pair_perm(8).tolist() == [0, 4, 1, 5, 2, 6, 3, 7]
    w = np.arange(2 * 4 * 3).reshape(8, 3)
    got = rope.interleave_rows(w, 2, 4)
    assert got[:, 0].tolist() == [0, 6, 3, 9, 12, 18, 15, 21]
    with pytest.raises(ValueError):
        rope.pair_perm(5)


def _rotate_half_host(x, cos, sin):
    """The host's RoPE on its own layout (pairs i, i + hd/2), torch fp64."""
    x = torch.from_numpy(x)
    c = torch.cat([cos, cos], -1)[:, None, :]
    s = torch.cat([sin, sin], -1)[:, None, :]
    half = x.shape[-1] // 2
    rot = torch.cat([-x[..., half:], x[..., :half]], -1)
    return (x * c + rot * s).numpy()


def test_adjacent_pairs_equal_rotate_half_under_the_permutation():
    rng = np.random.default_rng(3)
    S, H, hd, P = 5, 3, 64, 11
    table = wl.rope_table(S, hd, P)
    tf = codecs.bf16_to_f32(table).astype(np.float64)
    cos = torch.from_numpy(tf[:, 0::2].copy())
    sin = torch.from_numpy(tf[:, 1::2].copy())
    x = rng.standard_normal((S, H, hd))
    host = _rotate_half_host(x, cos, sin)
    perm = rope.pair_perm(hd)
    got = rope.rotate_pairs(x[..., perm], table)
    assert np.allclose(got, host[..., perm], rtol=0, atol=1e-12)


def test_special_angles_composition_and_norm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 1, 2))
    ident = _bf(np.array([[1.0, 0.0]]))
    assert np.array_equal(rope.rotate_pairs(x, ident), x)
    quarter = _bf(np.array([[0.0, 1.0]]))       # (a, b) -> (-b, a)
    assert np.array_equal(rope.rotate_pairs(x, quarter)[0, 0], [-x[0, 0, 1], x[0, 0, 0]])
    # two rotations by the same (cos, sin) pair compose like angles:
    # (c, s) twice is (c^2 - s^2, 2cs) (with c^2 + s^2 != 1 the composition
    # still holds for the unnormalised pair)
    r1 = _bf(np.array([[0.6, 0.8]]))
    c1, s1 = (float(v) for v in codecs.bf16_to_f32(r1)[0])
    twice = rope.rotate_pairs(rope.rotate_pairs(x, r1), r1)
    c2, s2 = c1 * c1 - s1 * s1, 2 * c1 * s1
    y = x[0, 0]
    want = [y[0] * c2 - y[1] * s2, y[1] * c2 + y[0] * s2]
    assert np.allclose(twice[0, 0], want, rtol=1e-14, atol=1e-14)
    # norm scales by c^2 + s^2
    r = rope.rotate_pairs(x, r1)
    assert math.isclose(float((r ** 2).sum()), float((x ** 2).sum()) * (c1 * c1 + s1 * s1),
                        rel_tol=1e-13)


def test_split_and_cache_placement_brute_force():
    rng = np.random.default_rng(5)
    S, nh, kv, hd, P, T = 3, 2, 1, 8, 4, 9
    width = (nh + 2 * kv) * hd
    qkv = _bf(rng.standard_normal((S, width + 5)))       # wider row stride
    table = wl.rope_table(S, hd, P)
    kc0 = _bf(rng.standard_normal((T, kv, hd)))
    vc0 = _bf(rng.standard_normal((T, kv, hd)))
    q, kc, vc = rope.qkv_split_rope_kvcache(qkv, table, nh, kv, hd, P, kc0, vc0)
    f = codecs.bf16_to_f32(qkv).astype(np.float64)
    tf = codecs.bf16_to_f32(table).astype(np.float64)

    def rot(vec, m):
        out = np.empty(hd)
        for i in range(hd // 2):
            a, b = vec[2 * i], vec[2 * i + 1]
            c, s = tf[m, 2 * i], tf[m, 2 * i + 1]
            out[2 * i], out[2 * i + 1] = a * c - b * s, b * c + a * s
        return codecs.f32_to_bf16(out.astype(np.float32))

    for m in range(S):
        for h in range(nh):
            assert np.array_equal(q[m, h], rot(f[m, h * hd:(h + 1) * hd], m))
        for h in range(kv):
            k0 = nh * hd + h * hd
            v0 = (nh + kv) * hd + h * hd
            assert np.array_equal(kc[P + m, h], rot(f[m, k0:k0 + hd], m))
            assert np.array_equal(vc[P + m, h], qkv[m, v0:v0 + hd])
    untouched = [r for r in range(T) if not P <= r < P + S]
    assert np.array_equal(kc[untouched], kc0[untouched])
    assert np.array_equal(vc[untouched], vc0[untouched])
    with pytest.raises(ValueError):
        rope.qkv_split_rope_kvcache(qkv, table, nh, kv, hd, 7, kc0, vc0)
