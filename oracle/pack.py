"""Joint-scale packing of sibling projections.

Test infrastructure only (see the package docstring).

Follows flashrt-structures 0.2.0, impls/qkv_pack/fp8_static.py
``_pack_weights`` (the same cast appears as ``_q8`` in
impls/modnorm_qkv_chain/fp8_ptok_table.py and as ``_amax_scale`` plus the
cast in impls/linear_proj/fp8_static.py): the sibling weights, each in
checkpoint layout ``[N_i, K]``, are concatenated along the output axis; one
scale ``s = max(fl32(amax|W| / 448), 1e-8)`` serves the whole group; the codes
are ``e4m3(clamp(fl32(W / s), -448, 448))``; the bias vector concatenates each
sibling's bias cast to bf16, or zeros for a sibling without one.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f32, e4m3_encode, E4M3_MAX


def pack_weights(W_bits_list, b_bits_list=None):
    """Returns ``(W8 [sum N_i, K] uint8, w_scale float32, bias_cat uint16
    [sum N_i], splits)``."""
    Ws = [np.asarray(w, dtype=np.uint16) for w in W_bits_list]
    K = Ws[0].shape[1]
    if any(w.shape[1] != K for w in Ws):
        raise ValueError("sibling K dims differ")
    W = bf16_to_f32(np.concatenate(Ws, axis=0))          # exact
    amax = np.float32(np.max(np.abs(W))) if W.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX))          # one fp32 rounding
    s = np.float32(max(s, np.float32(1e-8)))             # clamp(min=1e-8)
    q = (W / s).astype(np.float32)                       # fp32 division
    w8 = e4m3_encode(np.clip(q, -E4M3_MAX, E4M3_MAX))
    splits = [w.shape[0] for w in Ws]
    bias = []
    for i, n in enumerate(splits):
        b = None if b_bits_list is None else b_bits_list[i]
        bias.append(np.zeros(n, np.uint16) if b is None
                    else np.asarray(b, dtype=np.uint16).reshape(n))
    return w8, s, np.concatenate(bias), splits
