"""MI355X (gfx950) FP8 norm-quantize producers and packed sibling GEMM.

Thin ctypes binding over ``libfrt.so`` (built in-tree from ``csrc/`` by
``norm_quantize_packed_amd._build``). The Python functions carry the C ABI's
names and do argument marshalling only: torch tensors supply device
pointers, strides and the current HIP stream; every step of the computation
runs in the library's HIP kernels. There is no CPU fallback: if the library
is missing or fails to load, every call raises.

Tensor conventions: bf16 operands are ``torch.bfloat16`` (or 16-bit integer
views of bf16 bits), FP8 operands ``torch.float8_e4m3fn`` or ``torch.uint8``
code views, scales ``torch.float32`` device tensors of one element. Matrices
must be contiguous along their last dimension; the row stride is taken from
``stride(0)``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "FrtError", "load_library", "library_path",
    "frt_ada_norm_quant_fp8", "frt_ptok_table_norm_quant_fp8",
    "frt_pack_weights_fp8", "frt_packed_gemm_fp8_workspace_size",
    "frt_packed_gemm_fp8_split", "frt_geglu_quant_fp8",
    "frt_packed_gemm_fp8_geglu_quant", "frt_interleave_pairs_bf16",
    "frt_quantize_fp8_static", "frt_packed_gemm_bf16in_split",
    "frt_pack_weights_mxfp4", "frt_ada_norm_quant_mxfp4",
    "frt_packed_gemm_mxfp4_split", "frt_packed_gemm_mxfp4_geglu_quant",
    "frt_quantize_mxfp4", "frt_geglu_quant_mxfp4", "frt_packed_gemm_mxfp4_qkv_rope",
    "frt_packed_gemm_mxfp4_geglu_mxfp4",
    "frt_qkv_split_rope_kvcache", "frt_packed_gemm_fp8_qkv_rope",
    "frt_last_error", "frt_abi_version",
    "FRT_OK", "FRT_E_INVALID", "FRT_E_UNSUPPORTED", "FRT_E_HIP",
]

FRT_OK, FRT_E_INVALID, FRT_E_UNSUPPORTED, FRT_E_HIP = 0, -1, -2, -3
FRT_MAX_SPLITS = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "frt_last_error": (ctypes.c_char_p, []),
    "frt_abi_version": (_i32, []),
    "frt_ada_norm_quant_fp8": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _f32,
        _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p]),
    "frt_ptok_table_norm_quant_fp8": (_i32, [
        _p, _i64, _i64, _i32, _p, _i64, _p, _i64, _p, _p, _i32, _i32, _f32,
        _p, _i64, _p, _i64, _p]),
    "frt_pack_weights_fp8": (_i32, [
        _p, _i32, ctypes.POINTER(_i64), _i64, ctypes.POINTER(_p),
        ctypes.POINTER(_p), _p, _p, _p]),
    "frt_packed_gemm_fp8_workspace_size": (_sz, [_i64, _i64, _i64]),
    "frt_packed_gemm_fp8_split": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i32,
        ctypes.POINTER(_i64), ctypes.POINTER(_p), ctypes.POINTER(_i64), _i32,
        _p, _sz]),
    "frt_geglu_quant_fp8": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _i64, _p]),
    "frt_packed_gemm_fp8_geglu_quant": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _p, _p, _p, _i64]),
    "frt_interleave_pairs_bf16": (_i32, [_p, _i32, _i32, _i64, _p, _p]),
    "frt_quantize_fp8_static": (_i32, [_p, _i64, _i64, _p, _i64, _p, _p, _i64, _p]),
    "frt_pack_weights_mxfp4": (_i32, [
        _p, _i32, ctypes.POINTER(_i64), _i64, ctypes.POINTER(_p),
        ctypes.POINTER(_p), _p, _p, _p]),
    "frt_ada_norm_quant_mxfp4": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _f32,
        _p, _i64, _p, _i64, _p, _i64, _p, _i64]),
    "frt_packed_gemm_mxfp4_split": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _i32,
        ctypes.POINTER(_i64), ctypes.POINTER(_p), ctypes.POINTER(_i64), _i32]),
    "frt_packed_gemm_mxfp4_geglu_quant": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _p, _p, _i64]),
    "frt_quantize_mxfp4": (_i32, [_p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]),
    "frt_packed_gemm_mxfp4_geglu_mxfp4": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _i64]),
    "frt_packed_gemm_mxfp4_qkv_rope": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _p, _i32, _i32, _i32, _p, _p, _i64, _i64,
        _p, _p, _p]),
    "frt_geglu_quant_mxfp4": (_i32, [_p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64]),
    "frt_packed_gemm_bf16in_split": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i32,
        ctypes.POINTER(_i64), ctypes.POINTER(_p), ctypes.POINTER(_i64), _i32,
        _p, _sz]),
    "frt_qkv_split_rope_kvcache": (_i32, [
        _p, _i64, _i32, _i32, _i32, _p, _i64, _p, _i64, _i64, _p, _p, _p]),
    "frt_packed_gemm_fp8_qkv_rope": (_i32, [
        _p, _i64, _i64, _p, _i64, _p, _i32, _i32, _i32, _p, _p, _p, _p,
        _i64, _i64, _p, _p, _p]),
}


class FrtError(RuntimeError):
    """A refused or failed library call (status code + reason)."""

    def __init__(self, status: int, reason: str):
        super().__init__(f"frt status {status}: {reason}")
        self.status = status
        self.reason = reason


def library_path() -> str:
    return os.environ.get("FRT_LIBRARY", os.path.join(_HERE, "libfrt.so"))


def load_library() -> ctypes.CDLL:
    """Load libfrt.so (once). Raises if it is missing: there is no
    fallback path."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"frt: HIP library not built ({path} missing); run "
                "`python -m norm_quantize_packed_amd._build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def frt_last_error() -> str:
    return load_library().frt_last_error().decode()


def frt_abi_version() -> int:
    return load_library().frt_abi_version()


def _check(status: int):
    if status != FRT_OK:
        raise FrtError(status, frt_last_error())


# ------------------------------------------------------------ marshalling

def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _ld(t, rows_dim: int = 0) -> int:
    if t is None:
        return 0
    if t.dim() < 2:
        return 0
    if t.stride(-1) != 1:
        raise ValueError("frt: tensors must be contiguous along the last dim")
    return int(t.stride(rows_dim))


def _bf16_like(t, name):
    if t is None:
        return
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"frt: {name} must be bfloat16 (or 16-bit bits), "
                        f"got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"frt: {name} must be a device tensor")


def _u8_like(t, name):
    if t is None:
        return
    import torch
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.int8):
        raise TypeError(f"frt: {name} must be e4m3fn codes, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"frt: {name} must be a device tensor")


def _f32_like(t, name):
    if t is None:
        return
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"frt: {name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"frt: {name} must be a device tensor")


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------ entry points

def frt_ada_norm_quant_fp8(residual, mod, act_scale=None, *, x=None,
                           gate=None, weight=None, eps: float = 1e-6,
                           residual_out=None, out_fp8=None, gate_out=None,
                           y_f32=None, amax_out=None, M: Optional[int] = None,
                           stream=None) -> None:
    """Gated residual + AdaRMS + static FP8 (see include/frt.h).

    ``gate`` 1-D => one broadcast row; ``mod`` with one row (or 1-D) =>
    broadcast. ``M`` defaults to ``residual.shape[0]``."""
    for t, n in ((residual, "residual"), (mod, "mod"), (x, "x"),
                 (gate, "gate"), (weight, "weight"),
                 (residual_out, "residual_out"), (gate_out, "gate_out")):
        _bf16_like(t, n)
    _u8_like(out_fp8, "out_fp8")
    for t, n in ((act_scale, "act_scale"), (y_f32, "y_f32"),
                 (amax_out, "amax_out")):
        _f32_like(t, n)
    Mv = residual.shape[0] if M is None else int(M)
    D = residual.shape[-1]
    ld_mod = 0 if (mod.dim() == 1 or mod.shape[0] == 1) else _ld(mod)
    ld_gate = 0 if (gate is None or gate.dim() == 1 or gate.shape[0] == 1) \
        else _ld(gate)
    lib = load_library()
    _check(lib.frt_ada_norm_quant_fp8(
        _stream(stream), Mv, D, _ptr(residual), _ld(residual), _ptr(x),
        _ld(x), _ptr(gate), ld_gate, _ptr(weight), _ptr(mod), ld_mod,
        _ptr(act_scale), float(eps), _ptr(residual_out), _ld(residual_out),
        _ptr(out_fp8), _ld(out_fp8), _ptr(gate_out), _ld(gate_out),
        _ptr(y_f32), _ld(y_f32), _ptr(amax_out)))


def frt_ptok_table_norm_quant_fp8(x, temb, table, act_scale, shift_idx: int,
                                  scale_idx: int, *, eps: float = 1e-6,
                                  out_fp8=None, y_f32=None, amax_out=None,
                                  R: Optional[int] = None,
                                  stream=None) -> None:
    """Per-token-table no-affine adaptive LayerNorm + static FP8.

    ``temb`` is ``[R, C, D]`` (or ``[R, C*D]``), ``table`` ``[C, D]``."""
    _bf16_like(x, "x")
    _bf16_like(temb, "temb")
    _u8_like(out_fp8, "out_fp8")
    for t, n in ((table, "table"), (act_scale, "act_scale"),
                 (y_f32, "y_f32"), (amax_out, "amax_out")):
        _f32_like(t, n)
    Rv = x.shape[0] if R is None else int(R)
    D = x.shape[-1]
    C = table.shape[0]
    if temb.stride(-1) != 1:
        raise ValueError("frt: temb must be contiguous along D")
    if not table.is_contiguous():
        raise ValueError("frt: table must be contiguous")
    lib = load_library()
    _check(lib.frt_ptok_table_norm_quant_fp8(
        _stream(stream), Rv, D, C, _ptr(x), _ld(x), _ptr(temb),
        int(temb.stride(0)), _ptr(table), _ptr(act_scale), int(shift_idx),
        int(scale_idx), float(eps), _ptr(out_fp8), _ld(out_fp8),
        _ptr(y_f32), _ld(y_f32), _ptr(amax_out)))


def frt_pack_weights_fp8(weights: Sequence, biases: Optional[Sequence],
                         W8, w_scale, bias_cat=None, *, stream=None) -> None:
    """Joint-scale FP8 packing of sibling ``[N_i, K]`` bf16 weights."""
    n = len(weights)
    K = weights[0].shape[1]
    for i, w in enumerate(weights):
        _bf16_like(w, f"W_{i}")
        if not w.is_contiguous():
            raise ValueError("frt: sibling weights must be contiguous")
    _u8_like(W8, "W8")
    _f32_like(w_scale, "w_scale")
    _bf16_like(bias_cat, "bias_cat")
    Ns = (_i64 * n)(*[int(w.shape[0]) for w in weights])
    Ws = (_p * n)(*[_ptr(w) for w in weights])
    if biases is None:
        Bs = None
    else:
        for i, b in enumerate(biases):
            _bf16_like(b, f"b_{i}")
        Bs = (_p * n)(*[_ptr(b) for b in biases])
    lib = load_library()
    _check(lib.frt_pack_weights_fp8(_stream(stream), n, Ns, K, Ws, Bs,
                                    _ptr(W8), _ptr(w_scale), _ptr(bias_cat)))


def frt_packed_gemm_fp8_workspace_size(M: int, N_total: int, K: int) -> int:
    return int(load_library().frt_packed_gemm_fp8_workspace_size(M, N_total, K))


def frt_packed_gemm_fp8_split(x8, W8, act_scale, w_scale, outs: Sequence,
                              split_n: Sequence[int], bias_cat=None, *,
                              M: Optional[int] = None, workspace=None,
                              stream=None) -> None:
    """Packed FP8 GEMM + dequant + bias, each split written to ``outs[s]``
    (bf16 or float32 tensors ``[>= M, split_n[s]]``, any row stride)."""
    import torch
    _u8_like(x8, "x8")
    _u8_like(W8, "W8")
    _f32_like(act_scale, "act_scale")
    _f32_like(w_scale, "w_scale")
    _bf16_like(bias_cat, "bias_cat")
    n = len(split_n)
    if len(outs) != n:
        raise ValueError("frt: one output per split")
    dts = {o.dtype for o in outs}
    if dts == {torch.float32}:
        out_dtype = 1
    elif dts <= {torch.bfloat16, torch.int16, torch.uint16}:
        out_dtype = 0
    else:
        raise TypeError(f"frt: outputs must all be bf16 or all float32: {dts}")
    for o in outs:
        if not o.is_cuda:
            raise ValueError("frt: outputs must be device tensors")
    Mv = x8.shape[0] if M is None else int(M)
    K = x8.shape[1]
    N = W8.shape[0]
    ws_need = frt_packed_gemm_fp8_workspace_size(Mv, N, K)
    ws_ptr, ws_bytes = 0, 0
    if ws_need:
        # the caller owns every buffer: a plan that needs a workspace is
        # refused here rather than allocated behind the caller's back
        if workspace is None:
            raise ValueError(f"frt: this GEMM needs a device workspace of {ws_need} bytes "
                             "(frt_packed_gemm_fp8_workspace_size); pass workspace=")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    lib = load_library()
    _check(lib.frt_packed_gemm_fp8_split(
        _stream(stream), Mv, K, _ptr(x8), _ld(x8), _ptr(W8), N,
        _ptr(act_scale), _ptr(w_scale), _ptr(bias_cat), n,
        (_i64 * n)(*[int(s) for s in split_n]),
        (_p * n)(*[_ptr(o) for o in outs]),
        (_i64 * n)(*[_ld(o) for o in outs]), out_dtype, ws_ptr, ws_bytes))


def frt_geglu_quant_fp8(gu, H: int, act_scale=None, *, out_fp8=None,
                        y_f32=None, amax_out=None, M: Optional[int] = None,
                        stream=None) -> None:
    """GEGLU of the merged ``[M, >= 2H]`` bf16 gate|up rows + static FP8
    (see include/frt.h)."""
    _bf16_like(gu, "gu")
    _u8_like(out_fp8, "out_fp8")
    for t, n in ((act_scale, "act_scale"), (y_f32, "y_f32"),
                 (amax_out, "amax_out")):
        _f32_like(t, n)
    Mv = gu.shape[0] if M is None else int(M)
    lib = load_library()
    _check(lib.frt_geglu_quant_fp8(
        _stream(stream), Mv, int(H), _ptr(gu), _ld(gu), _ptr(act_scale),
        _ptr(out_fp8), _ld(out_fp8), _ptr(y_f32), _ld(y_f32),
        _ptr(amax_out)))


def frt_packed_gemm_fp8_geglu_quant(x8, W8, act_scale, w_scale, out_scale,
                                    out_fp8, bias_cat=None, *,
                                    M: Optional[int] = None,
                                    stream=None) -> None:
    """Merged gate/up FP8 GEMM (``W8`` = ``[2H, K]``, gate rows first) with
    the GEGLU quantiser as epilogue; ``out_fp8`` is ``[>= M, >= H]``."""
    _u8_like(x8, "x8")
    _u8_like(W8, "W8")
    _u8_like(out_fp8, "out_fp8")
    for t, n in ((act_scale, "act_scale"), (w_scale, "w_scale"),
                 (out_scale, "out_scale")):
        _f32_like(t, n)
    _bf16_like(bias_cat, "bias_cat")
    if W8.shape[0] % 2:
        raise ValueError("frt: W8 must hold 2H rows (gate, then up)")
    Mv = x8.shape[0] if M is None else int(M)
    lib = load_library()
    _check(lib.frt_packed_gemm_fp8_geglu_quant(
        _stream(stream), Mv, int(x8.shape[1]), _ptr(x8), _ld(x8), _ptr(W8),
        int(W8.shape[0] // 2), _ptr(act_scale), _ptr(w_scale),
        _ptr(bias_cat), _ptr(out_scale), _ptr(out_fp8), _ld(out_fp8)))


def frt_interleave_pairs_bf16(src, dst, nheads: int, hd: int, *,
                              stream=None) -> None:
    """Pack-time pair interleave of ``[nheads * hd, K]`` bf16 q or k rows."""
    _bf16_like(src, "src")
    _bf16_like(dst, "dst")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("frt: src and dst must be contiguous")
    _check(load_library().frt_interleave_pairs_bf16(
        _stream(stream), int(nheads), int(hd), int(src.shape[-1]), _ptr(src),
        _ptr(dst)))


def _cache_args(rope, q_out, k_cache, v_cache):
    for t, n in ((rope, "rope"), (q_out, "q_out"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _bf16_like(t, n)
        if not t.is_contiguous():
            raise ValueError(f"frt: {n} must be contiguous")


def frt_qkv_split_rope_kvcache(qkv, rope, nh: int, kv: int, hd: int, P: int,
                               q_out, k_cache, v_cache, *,
                               S: Optional[int] = None, stream=None) -> None:
    """Split the ``[S, (nh + 2kv) hd]`` QKV rows, rotate q/k by adjacent-pair
    RoPE, write ``q_out [S, nh, hd]`` and cache rows ``P .. P + S - 1`` of
    ``[T, kv, hd]`` caches."""
    _bf16_like(qkv, "qkv")
    _cache_args(rope, q_out, k_cache, v_cache)
    Sv = qkv.shape[0] if S is None else int(S)
    T = k_cache.numel() // (kv * hd)
    _check(load_library().frt_qkv_split_rope_kvcache(
        _stream(stream), Sv, int(nh), int(kv), int(hd), _ptr(qkv), _ld(qkv),
        _ptr(rope), int(P), int(T), _ptr(q_out), _ptr(k_cache), _ptr(v_cache)))


def frt_packed_gemm_fp8_qkv_rope(x8, W8, act_scale, w_scale, nh: int, kv: int,
                                 hd: int, rope, P: int, q_out, k_cache, v_cache,
                                 bias_cat=None, *, M: Optional[int] = None,
                                 stream=None) -> None:
    """Merged QKV FP8 GEMM with the split + RoPE + KV-cache epilogue."""
    _u8_like(x8, "x8")
    _u8_like(W8, "W8")
    for t, n in ((act_scale, "act_scale"), (w_scale, "w_scale")):
        _f32_like(t, n)
    _bf16_like(bias_cat, "bias_cat")
    _cache_args(rope, q_out, k_cache, v_cache)
    Mv = x8.shape[0] if M is None else int(M)
    T = k_cache.numel() // (kv * hd)
    _check(load_library().frt_packed_gemm_fp8_qkv_rope(
        _stream(stream), Mv, int(x8.shape[1]), _ptr(x8), _ld(x8), _ptr(W8),
        int(nh), int(kv), int(hd), _ptr(act_scale), _ptr(w_scale),
        _ptr(bias_cat), _ptr(rope), int(P), int(T), _ptr(q_out),
        _ptr(k_cache), _ptr(v_cache)))


def frt_quantize_fp8_static(x, act_scale=None, *, out_fp8=None, amax_out=None,
                            M: Optional[int] = None, stream=None) -> None:
    """Static per-tensor FP8 of a bf16 ``[M, D]`` tensor."""
    _bf16_like(x, "x")
    _u8_like(out_fp8, "out_fp8")
    for t, n in ((act_scale, "act_scale"), (amax_out, "amax_out")):
        _f32_like(t, n)
    Mv = x.shape[0] if M is None else int(M)
    _check(load_library().frt_quantize_fp8_static(
        _stream(stream), Mv, int(x.shape[-1]), _ptr(x), _ld(x), _ptr(act_scale),
        _ptr(out_fp8), _ld(out_fp8), _ptr(amax_out)))


def frt_packed_gemm_bf16in_split(x, x8, W8, act_scale, w_scale, outs: Sequence,
                                 split_n: Sequence[int], bias_cat=None, *,
                                 M: Optional[int] = None, stream=None) -> None:
    """bf16-input packed GEMM: ``x`` quantised into ``x8``, then
    ``frt_packed_gemm_fp8_split`` on it."""
    import torch
    _bf16_like(x, "x")
    _u8_like(x8, "x8")
    _u8_like(W8, "W8")
    _f32_like(act_scale, "act_scale")
    _f32_like(w_scale, "w_scale")
    _bf16_like(bias_cat, "bias_cat")
    n = len(split_n)
    if len(outs) != n:
        raise ValueError("frt: one output per split")
    dts = {o.dtype for o in outs}
    out_dtype = 1 if dts == {torch.float32} else 0
    Mv = x.shape[0] if M is None else int(M)
    K = x.shape[1]
    _check(load_library().frt_packed_gemm_bf16in_split(
        _stream(stream), Mv, K, _ptr(x), _ld(x), _ptr(x8), _ld(x8), _ptr(W8),
        int(W8.shape[0]), _ptr(act_scale), _ptr(w_scale), _ptr(bias_cat), n,
        (_i64 * n)(*[int(v) for v in split_n]), (_p * n)(*[_ptr(o) for o in outs]),
        (_i64 * n)(*[_ld(o) for o in outs]), out_dtype, 0, 0))


def frt_pack_weights_mxfp4(weights: Sequence, biases: Optional[Sequence], W4, S4,
                           bias_cat=None, *, stream=None) -> None:
    """MXFP4 packing of sibling ``[N_i, K]`` bf16 weights: codes ``W4``
    ``[sum N, K/2]`` and E8M0 scales ``S4`` ``[K/256, sum N, 8]``."""
    n = len(weights)
    K = weights[0].shape[1]
    for i, w in enumerate(weights):
        _bf16_like(w, f"W_{i}")
        if not w.is_contiguous():
            raise ValueError("frt: sibling weights must be contiguous")
    _u8_like(W4, "W4")
    _u8_like(S4, "S4")
    _bf16_like(bias_cat, "bias_cat")
    Ns = (_i64 * n)(*[int(w.shape[0]) for w in weights])
    Ws = (_p * n)(*[_ptr(w) for w in weights])
    Bs = None if biases is None else (_p * n)(*[_ptr(b) for b in biases])
    _check(load_library().frt_pack_weights_mxfp4(_stream(stream), n, Ns, K, Ws, Bs,
                                                  _ptr(W4), _ptr(S4), _ptr(bias_cat)))


def frt_ada_norm_quant_mxfp4(residual, mod, out_fp4, out_scale, *, x=None,
                             gate=None, weight=None, eps: float = 1e-6,
                             residual_out=None, gate_out=None,
                             M: Optional[int] = None, stream=None) -> None:
    """Gated residual + AdaRMS with an MXFP4 output (codes ``[M, D/2]``,
    scales ``[D/256, rows, 8]``; the run stride is ``stride(0)``)."""
    for t, n in ((residual, "residual"), (mod, "mod"), (x, "x"),
                 (gate, "gate"), (weight, "weight"),
                 (residual_out, "residual_out"), (gate_out, "gate_out")):
        _bf16_like(t, n)
    _u8_like(out_fp4, "out_fp4")
    _u8_like(out_scale, "out_scale")
    Mv = residual.shape[0] if M is None else int(M)
    D = residual.shape[-1]
    ld_mod = 0 if (mod.dim() == 1 or mod.shape[0] == 1) else _ld(mod)
    ld_gate = 0 if (gate is None or gate.dim() == 1 or gate.shape[0] == 1) \
        else _ld(gate)
    _check(load_library().frt_ada_norm_quant_mxfp4(
        _stream(stream), Mv, D, _ptr(residual), _ld(residual), _ptr(x), _ld(x),
        _ptr(gate), ld_gate, _ptr(weight), _ptr(mod), ld_mod, float(eps),
        _ptr(residual_out), _ld(residual_out), _ptr(out_fp4), _ld(out_fp4),
        _ptr(out_scale), _ld(out_scale), _ptr(gate_out), _ld(gate_out)))


def frt_packed_gemm_mxfp4_split(x4, xs, W4, S4, outs: Sequence,
                                split_n: Sequence[int], bias_cat=None, *,
                                M: Optional[int] = None, stream=None) -> None:
    """Packed GEMM on MXFP4 operands (codes ``x4 [M, K/2]``, scales
    ``xs [K/256, rows, 8]``; ``W4``/``S4`` from ``frt_pack_weights_mxfp4``)."""
    import torch
    for t, nme in ((x4, "x4"), (xs, "xs"), (W4, "W4"), (S4, "S4")):
        _u8_like(t, nme)
    _bf16_like(bias_cat, "bias_cat")
    n = len(split_n)
    if len(outs) != n:
        raise ValueError("frt: one output per split")
    out_dtype = 1 if {o.dtype for o in outs} == {torch.float32} else 0
    Mv = x4.shape[0] if M is None else int(M)
    K = int(W4.shape[1]) * 2
    _check(load_library().frt_packed_gemm_mxfp4_split(
        _stream(stream), Mv, K, _ptr(x4), _ld(x4), _ptr(xs), _ld(xs), _ptr(W4),
        _ptr(S4), int(W4.shape[0]), _ptr(bias_cat), n,
        (_i64 * n)(*[int(v) for v in split_n]), (_p * n)(*[_ptr(o) for o in outs]),
        (_i64 * n)(*[_ld(o) for o in outs]), out_dtype))


def frt_packed_gemm_mxfp4_geglu_quant(x4, xs, W4, S4, out_scale, out_fp8,
                                      bias_cat=None, *, M: Optional[int] = None,
                                      stream=None) -> None:
    """Merged gate/up GEMM on MXFP4 operands (``W4`` = ``[2H, K/2]``, gate
    rows first, ``S4`` its ``[K/256, 2H, 8]`` scales) with the GEGLU
    quantiser as epilogue; ``out_fp8`` is ``[>= M, >= H]`` e4m3fn codes."""
    for t, nme in ((x4, "x4"), (xs, "xs"), (W4, "W4"), (S4, "S4"), (out_fp8, "out_fp8")):
        _u8_like(t, nme)
    _f32_like(out_scale, "out_scale")
    _bf16_like(bias_cat, "bias_cat")
    if W4.shape[0] % 2:
        raise ValueError("frt: W4 must hold 2H rows (gate, then up)")
    Mv = x4.shape[0] if M is None else int(M)
    _check(load_library().frt_packed_gemm_mxfp4_geglu_quant(
        _stream(stream), Mv, int(W4.shape[1]) * 2, _ptr(x4), _ld(x4), _ptr(xs), _ld(xs),
        _ptr(W4), _ptr(S4), int(W4.shape[0] // 2), _ptr(bias_cat), _ptr(out_scale),
        _ptr(out_fp8), _ld(out_fp8)))


def frt_quantize_mxfp4(x, out_fp4, out_scale, *, M: Optional[int] = None,
                       stream=None) -> None:
    """Dynamic MXFP4 of a bf16 ``x [M, D]``: codes into ``out_fp4
    [M, D/2]``, scales into ``out_scale [D/256, rows, 8]``."""
    _bf16_like(x, "x")
    _u8_like(out_fp4, "out_fp4")
    _u8_like(out_scale, "out_scale")
    Mv = x.shape[0] if M is None else int(M)
    _check(load_library().frt_quantize_mxfp4(
        _stream(stream), Mv, int(x.shape[1]), _ptr(x), _ld(x), _ptr(out_fp4), _ld(out_fp4),
        _ptr(out_scale), _ld(out_scale)))


def frt_geglu_quant_mxfp4(gu, H: int, out_fp4, out_scale, *,
                          M: Optional[int] = None, stream=None) -> None:
    """GEGLU of a bf16 gate|up buffer ``gu [M, >= 2H]`` quantised to MXFP4:
    codes into ``out_fp4 [M, H/2]``, scales into ``out_scale [H/256, rows, 8]``."""
    _bf16_like(gu, "gu")
    _u8_like(out_fp4, "out_fp4")
    _u8_like(out_scale, "out_scale")
    Mv = gu.shape[0] if M is None else int(M)
    _check(load_library().frt_geglu_quant_mxfp4(
        _stream(stream), Mv, int(H), _ptr(gu), _ld(gu), _ptr(out_fp4), _ld(out_fp4),
        _ptr(out_scale), _ld(out_scale)))


def frt_packed_gemm_mxfp4_qkv_rope(x4, xs, W4, S4, nh: int, kv: int, hd: int, rope,
                                   P: int, q_out, k_cache, v_cache, bias_cat=None, *,
                                   M: Optional[int] = None, stream=None) -> None:
    """Merged QKV GEMM on MXFP4 operands with the split + RoPE + KV-cache
    epilogue (q and k weight rows pair-interleaved before packing)."""
    for t, nme in ((x4, "x4"), (xs, "xs"), (W4, "W4"), (S4, "S4")):
        _u8_like(t, nme)
    _bf16_like(bias_cat, "bias_cat")
    _cache_args(rope, q_out, k_cache, v_cache)
    Mv = x4.shape[0] if M is None else int(M)
    T = k_cache.numel() // (kv * hd)
    _check(load_library().frt_packed_gemm_mxfp4_qkv_rope(
        _stream(stream), Mv, int(W4.shape[1]) * 2, _ptr(x4), _ld(x4), _ptr(xs), _ld(xs),
        _ptr(W4), _ptr(S4), int(nh), int(kv), int(hd), _ptr(bias_cat), _ptr(rope), int(P),
        int(T), _ptr(q_out), _ptr(k_cache), _ptr(v_cache)))


def frt_packed_gemm_mxfp4_geglu_mxfp4(x4, xs, W4, S4, out_fp4, out_scale, bias_cat=None, *,
                                      M: Optional[int] = None, stream=None) -> None:
    """Merged gate/up GEMM on MXFP4 operands with the GEGLU quantised to
    MXFP4 in its epilogue: codes into ``out_fp4 [M, H/2]``, scales into
    ``out_scale [H/256, rows, 8]``."""
    for t, nme in ((x4, "x4"), (xs, "xs"), (W4, "W4"), (S4, "S4"), (out_fp4, "out_fp4"),
                   (out_scale, "out_scale")):
        _u8_like(t, nme)
    _bf16_like(bias_cat, "bias_cat")
    if W4.shape[0] % 2:
        raise ValueError("frt: W4 must hold 2H rows (gate, then up)")
    Mv = x4.shape[0] if M is None else int(M)
    _check(load_library().frt_packed_gemm_mxfp4_geglu_mxfp4(
        _stream(stream), Mv, int(W4.shape[1]) * 2, _ptr(x4), _ld(x4), _ptr(xs), _ld(xs),
        _ptr(W4), _ptr(S4), int(W4.shape[0] // 2), _ptr(bias_cat), _ptr(out_fp4), _ld(out_fp4),
        _ptr(out_scale), _ld(out_scale)))
