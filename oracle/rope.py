"""QKV split + adjacent-pair RoPE + KV-cache write, the consumer of the
merged QKV GEMM.

Test infrastructure only (see the package docstring).

Sources (flashrt-structures 0.2.0 wheel pages, impls/adarms_stack/
fp8_chain.py):
- module docstring: the host rotates pairs (i, i + hd/2) (rotate-half);
  the split kernel rotates adjacent pairs, so the q and k projection rows
  are permuted when the weights are packed (``_interleave_rows``, the
  ``kperm`` gather: position 2i takes dimension i, position 2i + 1 takes
  dimension i + hd/2); V keeps host order;
- ``_build_rope``: the rope table is bf16 ``[S, hd]`` with the pair's
  cosine at even and its sine at odd positions (``rope[:, 0::2] = cos``,
  ``rope[:, 1::2] = sin`` of the first half);
- ``_make_run``: ``qkv_split_rope_kvcache_bf16(qkv3, rope, nh, kv, hd, P,
  q_out=q, k_cache=kc, v_cache=vc, max_seq_len=T)`` on the merged QKV
  output viewed ``[1, S, (nh + 2 kv) hd]``, with the suffix K/V written
  behind the P prefix rows of ``[1, T, kv, hd]`` caches, T = P + S
  (``total_keys = p_used + S``).

Readings where the pages are silent:
- the rotation of an adjacent pair (a, b) with (c, s) = (cos, sin) is the
  standard one, a' = a c - b s, b' = b c + a s (what rotate-half computes
  on the host layout);
- q, k, v and the table enter as bf16 values; the rotation is exact in
  real arithmetic and rounded once to bf16 (via fp32, like every bf16
  output here: both products of two bf16 values are exact in fp32, so an
  FMA-based kernel forms the same fp32 value);
- row m of the call is token m: it uses rope row m, writes q_out row m and
  cache row P + m; cache rows outside [P, P + S) are not touched.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f32, f32_to_bf16


def pair_perm(hd):
    """``kperm``: position 2i <- dimension i, 2i + 1 <- dimension i + hd/2."""
    if hd % 2:
        raise ValueError("head dim must be even")
    half = hd // 2
    p = np.empty(hd, dtype=np.int64)
    p[0::2] = np.arange(half)
    p[1::2] = np.arange(half, hd)
    return p


def interleave_rows(w_bits, nheads, hd):
    """Permute the rows of a ``[nheads * hd, K]`` projection within each
    head by ``pair_perm`` (the pack-time permutation of q and k)."""
    w = np.asarray(w_bits)
    if w.shape[0] != nheads * hd:
        raise ValueError("rows must be nheads * hd")
    idx = (np.arange(nheads)[:, None] * hd + pair_perm(hd)[None, :]).reshape(-1)
    return w[idx]


def rotate_pairs(x, rope_bits):
    """Adjacent-pair rotation in float64. ``x`` is ``[S, heads, hd]`` (float),
    ``rope_bits`` bf16 ``[S, hd]`` (cos at even, sin at odd positions)."""
    x = np.asarray(x, dtype=np.float64)
    r = bf16_to_f32(np.asarray(rope_bits, dtype=np.uint16)).astype(np.float64)
    c = r[:, None, 0::2]
    s = r[:, None, 1::2]
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def qkv_split_rope_kvcache(qkv_bits, rope_bits, nh, kv, hd, P, k_cache_bits,
                           v_cache_bits):
    """The split + RoPE + cache write on bf16 bits.

    ``qkv_bits`` ``[S, (nh + 2 kv) hd]`` (row stride may be wider);
    ``rope_bits`` ``[S, hd]``; caches ``[T, kv, hd]`` (copied, then rows
    ``P .. P + S - 1`` overwritten). Returns ``(q_out [S, nh, hd],
    k_cache, v_cache)`` as bf16 bits."""
    qkv = np.asarray(qkv_bits, dtype=np.uint16)
    S = qkv.shape[0]
    nq, nk = nh * hd, kv * hd
    if qkv.shape[1] < nq + 2 * nk:
        raise ValueError("qkv row too short")
    kc = np.array(k_cache_bits, dtype=np.uint16, copy=True)
    vc = np.array(v_cache_bits, dtype=np.uint16, copy=True)
    if P < 0 or P + S > kc.shape[0]:
        raise ValueError("cache rows P .. P + S - 1 out of range")
    f = bf16_to_f32(qkv).astype(np.float64)
    q = f[:, :nq].reshape(S, nh, hd)
    k = f[:, nq:nq + nk].reshape(S, kv, hd)
    q_out = f32_to_bf16(rotate_pairs(q, rope_bits).astype(np.float32))
    kc[P:P + S] = f32_to_bf16(rotate_pairs(k, rope_bits).astype(np.float32))
    vc[P:P + S] = qkv[:, nq + nk:nq + 2 * nk].reshape(S, kv, hd)
    return q_out, kc, vc
