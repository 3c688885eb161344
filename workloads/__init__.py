"""Seeded synthetic workloads for the norm-quantize producers and the packed
FP8 GEMM.

This module only draws random inputs and knows the five workload shapes. It
holds none of the method's arithmetic: no normalisation, no quantisation, no
GEMM. Both the CPU oracle tests and the GPU path (tests, bench) take their
inputs from here, so that the two sides see the same bits.

Every floating-point tensor is drawn in fp32 from a NumPy ``default_rng``
(PCG64) stream keyed by ``(seed, tensor id)`` and, where the kernels take
bf16, converted to bf16 bit patterns (``uint16``) by torch's CPU cast
(round to nearest even). The per-token table stays fp32.

Seeds per workload ``c`` (1..5): data ``1000 + c``, calibration batch
``2000 + c`` (same shapes and distributions as the data), weights and biases
``3000 + c``.

The workloads follow the pages' hosts: the AdaRMS decoder chain of
flashrt-structures 0.2.0 (impls/adarms_stack/fp8_chain.py, the fused
gated-residual AdaRMS producer feeding the merged QKV and gate/up GEMMs) and
the video-DiT per-token-table block (impls/modnorm_qkv_chain/fp8_ptok_table.py,
``PerTokenModChainBlock``), with the packed sibling weights of
impls/qkv_pack/fp8_static.py.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

EPS = 1e-6
_CHUNK = 1 << 24  # elements drawn per RNG call (bounds host memory)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: producer form, shapes, GEMM groups."""

    cid: int
    name: str
    form: str                    # "adarms" or "ptok"
    rows: int                    # producer rows (tokens, B*M for ptok)
    D: int                       # hidden size (= GEMM K)
    gemms: Tuple[Tuple[int, ...], ...]   # per producer site: sibling widths
    bias: bool                   # GEMM biases present
    w_std: float                 # weight standard deviation
    shift_idx: int = 0           # ptok chunk selection
    scale_idx: int = 1
    sites: int = 1               # chained AdaRMS producer sites
    m_sweep: Tuple[int, ...] = ()  # small-M timing sweep (latency band)

    @property
    def n_total(self) -> Tuple[int, ...]:
        return tuple(sum(g) for g in self.gemms)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "adarms_qkv_m16_d512", "adarms", 16, 512,
                ((512, 128, 128),), False, 0.02),
    2: Workload(2, "adarms_decoder_m256_d2048", "adarms", 256, 2048,
                ((2048, 256, 256), (8192, 8192)), False, 0.02, sites=2),
    3: Workload(3, "ptok_dit_qkv_b2_m4096_d3072", "ptok", 8192, 3072,
                ((3072, 3072, 3072),), True, 0.02, shift_idx=0, scale_idx=1),
    4: Workload(4, "adarms_small_m_d4096", "adarms", 64, 4096,
                ((4096, 1024, 1024),), False, 0.02,
                m_sweep=(1, 2, 4, 8, 16, 32, 64)),
    5: Workload(5, "ptok_ffn_gateup_m2048_d16384", "ptok", 2048, 16384,
                ((16384, 16384),), False, 1.0, shift_idx=3, scale_idx=4),
}

# small bit-level helpers -------------------------------------------------


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16) via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rng(seed: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor])


def normal_bf16(seed: int, tensor: int, shape: Sequence[int], std: float,
                out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bits of N(0, std^2) drawn in fp32, chunked to bound memory."""
    rng = _rng(seed, tensor)
    n = int(np.prod(shape))
    flat = np.empty(n, np.uint16) if out is None else out.reshape(-1)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        flat[lo:hi] = to_bf16_bits(v)
    return flat.reshape(shape)


def student_t_bf16(seed: int, tensor: int, shape: Sequence[int],
                   dof: float) -> np.ndarray:
    """bf16 bits of a Student-t(dof) draw (heavy-tailed activations)."""
    rng = _rng(seed, tensor)
    n = int(np.prod(shape))
    flat = np.empty(n, np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        v = rng.standard_t(dof, hi - lo).astype(np.float32)
        flat[lo:hi] = to_bf16_bits(v)
    return flat.reshape(shape)


def normal_f32(seed: int, tensor: int, shape: Sequence[int],
               std: float) -> np.ndarray:
    rng = _rng(seed, tensor)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v.reshape(shape)


def _with_outliers(seed: int, tensor: int, shape, channels, factor):
    """N(0,1) fp32 rows with the given channels scaled by ``factor``."""
    rng = _rng(seed, tensor)
    v = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    v = v.reshape(shape)
    v[:, channels] *= np.float32(factor)
    return to_bf16_bits(v)


# producer inputs ---------------------------------------------------------


def producer_inputs(cid: int, calib: bool = False,
                    rows: Optional[int] = None) -> dict:
    """Producer inputs of workload ``cid`` (the calibration batch if
    ``calib``), as bf16 bit arrays / fp32 arrays.

    AdaRMS workloads return ``residual``, ``x``, ``gate`` (``[D]`` broadcast
    row or ``[rows, D]``), ``mod`` (``[1, 3D]`` = scale | shift | gate) per
    site. Chained sites (workload 2) list the second site's ``x``, ``mod`` and
    the rule for its residual (the first site's residual output) and gate (the
    first site's mod-row gate chunk).

    ptok workloads return ``x [R, D]``, ``temb [R, 6, D]``, ``table [6, D]``.
    """
    w = WORKLOADS[cid]
    seed = (2000 if calib else 1000) + cid
    R = w.rows if rows is None else rows
    D = w.D
    out: dict = {"cid": cid, "rows": R, "D": D, "eps": EPS}
    if w.form == "ptok":
        if cid == 3:
            out["x"] = normal_bf16(seed, 0, (R, D), 1.0)
            out["temb"] = normal_bf16(seed, 1, (R, 6, D), 0.1)
            out["table"] = normal_f32(seed, 2, (6, D), 0.1)
        else:
            out["x"] = student_t_bf16(seed, 0, (R, D), 3.0)
            out["temb"] = normal_bf16(seed, 1, (R, 6, D), 1.0)
            out["table"] = normal_f32(seed, 2, (6, D), 1.0)
        out["shift_idx"], out["scale_idx"] = w.shift_idx, w.scale_idx
        return out
    if cid == 1:
        out["residual"] = normal_bf16(seed, 0, (R, D), 1.0)
        out["x"] = normal_bf16(seed, 1, (R, D), 1.0)
        out["mod"] = normal_bf16(seed, 2, (1, 3 * D), 0.1)
        # the previous site's mod row: its gate chunk is this site's
        # broadcast prev_gate
        prev = normal_bf16(seed, 3, (1, 3 * D), 0.1)
        out["gate"] = prev[0, 2 * D:3 * D].copy()
    elif cid == 2:
        ch = np.sort(_rng(seed, 99).choice(D, 4, replace=False))
        out["outlier_channels"] = ch
        out["residual"] = _with_outliers(seed, 0, (R, D), ch, 20.0)
        out["x"] = _with_outliers(seed, 1, (R, D), ch, 20.0)
        out["gate"] = normal_bf16(seed, 2, (D,), 0.1)
        out["mod"] = normal_bf16(seed, 3, (1, 3 * D), 0.1)
        out["x2"] = _with_outliers(seed, 4, (R, D), ch, 20.0)
        out["mod2"] = normal_bf16(seed, 5, (1, 3 * D), 0.1)
    elif cid == 4:
        full = 64
        out["residual"] = normal_bf16(seed, 0, (full, D), 1.0)[:R].copy()
        out["x"] = normal_bf16(seed, 1, (full, D), 1.0)[:R].copy()
        out["gate"] = normal_bf16(seed, 2, (full, D), 0.5)[:R].copy()
        out["mod"] = normal_bf16(seed, 3, (1, 3 * D), 0.1)
    else:
        raise ValueError(cid)
    return out


def weights(cid: int, site: int = 0) -> dict:
    """Sibling weights ``W_i`` (bf16 bits, ``[N_i, K]`` checkpoint layout)
    and biases ``b_i`` (bf16 bits or None) of workload ``cid``'s GEMM at
    producer site ``site``."""
    w = WORKLOADS[cid]
    seed = 3000 + cid
    widths = w.gemms[site]
    Ws, bs = [], []
    for i, n in enumerate(widths):
        Ws.append(normal_bf16(seed, 10 * site + i, (n, w.D), w.w_std))
        bs.append(normal_bf16(seed, 100 + 10 * site + i, (n,), 0.02)
                  if w.bias else None)
    return {"W": Ws, "b": bs, "splits": widths}


# The FFN tail after a gate/up GEMM (workloads 2 and 5): the down
# projection [D, H] that consumes the GEGLU output, drawn like the
# workload's other weights (bias-free).
FFN_HIDDEN: Dict[int, int] = {2: 8192, 5: 16384}


def down_weights(cid: int) -> np.ndarray:
    """Down-projection weight of workload ``cid`` as bf16 bits ``[D, H]``
    (checkpoint layout, H contiguous)."""
    w = WORKLOADS[cid]
    H = FFN_HIDDEN[cid]
    return normal_bf16(3000 + cid, 50, (w.D, H), w.w_std)


# The attention heads behind workload 2's merged QKV (2048 | 256 | 256 =
# 8 query heads and one KV head of 256), and the KV-cache geometry of the
# suffix pass: P prefix rows already cached, the 256 suffix tokens written
# behind them (T = P + S rows).
# Tensor parallelism over the GEMM's output columns: the column group a
# rank's share of every sibling must keep whole (one 128-wide attention head
# of the QKV projection; a 128-column group of the FFN hidden size).
TP_UNIT: Dict[int, int] = {3: 128, 5: 128}


def tp_shard(ws: dict, tp: int, rank: int = 0, unit: int = 128) -> dict:
    """Rank ``rank``'s share of ``weights()`` when the packed GEMM is split
    over ``tp`` GPUs by output columns: rows ``[rank*n/tp, (rank+1)*n/tp)``
    of every sibling ``W_i`` (``[n, K]``) and of its bias. Every ``n`` must
    be a multiple of ``tp * unit``."""
    Ws, bs, widths = [], [], []
    for W, b, n in zip(ws["W"], ws["b"], ws["splits"]):
        if n % (tp * unit):
            raise ValueError(f"sibling width {n} does not split into {tp} groups of {unit}-column units")
        m = n // tp
        Ws.append(np.ascontiguousarray(W[rank * m:(rank + 1) * m]))
        bs.append(None if b is None else np.ascontiguousarray(b[rank * m:(rank + 1) * m]))
        widths.append(m)
    return {"W": Ws, "b": bs, "splits": tuple(widths)}


QKV_HEADS: Dict[int, Tuple[int, int, int]] = {2: (8, 1, 256)}
ROPE_PREFIX: Dict[int, int] = {2: 768}


def o_proj_inputs(cid: int, calib: bool = False) -> dict:
    """The O projection of workload ``cid``'s attention heads: a seeded
    attention output ``att`` (bf16 ``[rows, nh*hd]``, N(0,1); the
    calibration batch with ``calib``) and the weight ``W_o`` (bf16
    ``[D, nh*hd]``, drawn like the workload's other weights, no bias)."""
    w = WORKLOADS[cid]
    nh, kv, hd = QKV_HEADS[cid]
    seed = (2000 if calib else 1000) + cid
    return {"att": normal_bf16(seed, 70, (w.rows, nh * hd), 1.0),
            "W_o": normal_bf16(3000 + cid, 60, (w.D, nh * hd), w.w_std)}


def rope_table(S: int, hd: int, P: int, base: float = 10000.0) -> np.ndarray:
    """bf16 bits ``[S, hd]`` of the rotary table for positions P .. P + S - 1:
    the cosine of pair i at column 2i and its sine at 2i + 1, angle
    ``pos * base^(-2i / hd)`` (the standard rotary frequencies)."""
    half = hd // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = (P + np.arange(S, dtype=np.float64))[:, None] * inv[None, :]
    t = np.empty((S, hd), dtype=np.float32)
    t[:, 0::2] = np.cos(ang)
    t[:, 1::2] = np.sin(ang)
    return to_bf16_bits(t)


def random_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Free-form helper for edge-case tests."""
    return normal_bf16(seed, 7, shape, std)


def random_codes(seed: int, shape) -> np.ndarray:
    """Uniformly random finite e4m3fn codes (NaN codes 0x7F/0xFF excluded)."""
    rng = _rng(seed, 11)
    c = rng.integers(0, 254, size=shape, dtype=np.int64)
    c = c + (c >= 127)          # skip 0x7F
    return c.astype(np.uint8)
