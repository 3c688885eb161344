"""The C ABI without a GPU: the library loads, exports every entry point
include/frt.h declares, and refuses out-of-contract calls on the host before
any HIP call (fake, never dereferenced device addresses are passed)."""

import ctypes
import os
import re

import pytest

import norm_quantize_packed_amd as frt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "frt.h")

FAKE = 0x7f0000000000       # a 16-byte-aligned address no call may touch
MB = 1 << 20


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(frt_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(frt.library_path()):
        pytest.fail("libfrt.so is not built; run python -m "
                    "norm_quantize_packed_amd._build")
    return frt.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"frt_ada_norm_quant_fp8", "frt_ptok_table_norm_quant_fp8",
            "frt_pack_weights_fp8", "frt_packed_gemm_fp8_split",
            "frt_packed_gemm_fp8_workspace_size",
            "frt_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.frt_abi_version() == 1


def _ada(lib, M=4, D=512, **kw):
    a = dict(stream=None, M=M, D=D, residual=FAKE, ld_res=D, x=FAKE + MB,
             ld_x=D, gate=FAKE + 2 * MB, ld_gate=0, weight=None,
             mod=FAKE + 3 * MB, ld_mod=0, act_scale=FAKE + 4 * MB, eps=1e-6,
             residual_out=FAKE + 5 * MB, ld_rout=D, out_fp8=FAKE + 6 * MB,
             ld_out=D, gate_out=None, ld_gout=0, y_f32=None, ld_y=0,
             amax_out=None)
    a.update(kw)
    return lib.frt_ada_norm_quant_fp8(*a.values())


def test_ada_refusals(lib):
    assert _ada(lib, D=500) == frt.FRT_E_INVALID
    assert "D=500" in frt.frt_last_error()
    assert _ada(lib, D=16386) == frt.FRT_E_INVALID
    assert _ada(lib, D=513) == frt.FRT_E_INVALID
    assert _ada(lib, M=-1) == frt.FRT_E_INVALID
    assert _ada(lib, residual=None) == frt.FRT_E_INVALID
    assert _ada(lib, act_scale=None) == frt.FRT_E_INVALID
    assert _ada(lib, ld_res=100) == frt.FRT_E_INVALID
    assert _ada(lib, ld_mod=700) == frt.FRT_E_INVALID
    assert _ada(lib, out_fp8=None, residual_out=None) == frt.FRT_E_INVALID
    # an output overlapping an input (other than the exact in-place residual)
    assert _ada(lib, out_fp8=FAKE + MB + 64) == frt.FRT_E_INVALID
    assert "overlaps" in frt.frt_last_error()
    assert _ada(lib, residual_out=FAKE + 64) == frt.FRT_E_INVALID
    # misaligned for every path
    assert _ada(lib, residual=FAKE + 1) == frt.FRT_E_INVALID


def test_ada_zero_rows_is_noop(lib):
    assert _ada(lib, M=0) == frt.FRT_OK
    # exact in-place residual passes validation (checked with M = 0)
    assert _ada(lib, M=0, residual_out=FAKE) == frt.FRT_OK
    assert frt.frt_last_error() == ""


def _ptok(lib, R=4, D=512, C=6, **kw):
    a = dict(stream=None, R=R, D=D, C=C, x=FAKE, ld_x=D, temb=FAKE + MB,
             ld_temb=C * D, table=FAKE + 20 * MB, act_scale=FAKE + 21 * MB,
             shift_idx=0, scale_idx=1, eps=1e-6, out_fp8=FAKE + 22 * MB,
             ld_out=D, y_f32=None, ld_y=0, amax_out=None)
    a.update(kw)
    return lib.frt_ptok_table_norm_quant_fp8(*a.values())


def test_ptok_refusals(lib):
    assert _ptok(lib, C=5) == frt.FRT_E_INVALID
    assert "6-chunk" in frt.frt_last_error()
    assert _ptok(lib, D=256) == frt.FRT_E_INVALID
    assert _ptok(lib, shift_idx=6) == frt.FRT_E_INVALID
    assert _ptok(lib, scale_idx=-1) == frt.FRT_E_INVALID
    assert _ptok(lib, ld_temb=512) == frt.FRT_E_INVALID
    assert _ptok(lib, temb=None) == frt.FRT_E_INVALID
    assert _ptok(lib, out_fp8=FAKE + MB + 512) == frt.FRT_E_INVALID
    assert _ptok(lib, R=0) == frt.FRT_OK


def _gemm(lib, M=16, K=512, splits=(512, 128, 128), N=None, outs=None,
          lds=None, **kw):
    n = len(splits)
    N = sum(splits) if N is None else N
    outs = outs or [FAKE + (40 + 4 * i) * MB for i in range(n)]
    lds = lds or list(splits)
    a = dict(stream=None, M=M, K=K, x8=FAKE, ld_x=K, W8=FAKE + MB, N=N,
             act_scale=FAKE + 30 * MB, w_scale=FAKE + 31 * MB, bias=None,
             n_split=n, split_n=(ctypes.c_int64 * n)(*splits),
             out=(ctypes.c_void_p * n)(*outs),
             ld_out=(ctypes.c_int64 * n)(*lds), out_dtype=0,
             ws=FAKE + 100 * MB, ws_bytes=16 * MB)
    a.update(kw)
    return lib.frt_packed_gemm_fp8_split(*a.values())


def test_gemm_refusals(lib):
    assert _gemm(lib, N=700) == frt.FRT_E_INVALID
    assert "sum" in frt.frt_last_error()
    assert _gemm(lib, K=256) == frt.FRT_E_INVALID
    assert _gemm(lib, K=520) == frt.FRT_E_UNSUPPORTED
    assert _gemm(lib, ld_x=520) == frt.FRT_E_INVALID
    assert _gemm(lib, x8=FAKE + 8) == frt.FRT_E_INVALID
    assert _gemm(lib, out_dtype=2) == frt.FRT_E_INVALID
    assert _gemm(lib, splits=(768,), lds=[100]) == frt.FRT_E_INVALID
    assert _gemm(lib, splits=(768, 0)) == frt.FRT_E_INVALID
    assert _gemm(lib, splits=tuple([1] * 17)) == frt.FRT_E_INVALID
    # overlapping split outputs
    o = FAKE + 40 * MB
    assert _gemm(lib, outs=[o, o + 512, o + 2 * MB]) == frt.FRT_E_INVALID
    assert "overlap" in frt.frt_last_error()
    # an output over an input
    assert _gemm(lib, outs=[FAKE + MB, o + MB, o + 2 * MB]) == frt.FRT_E_INVALID


def test_gemm_zero_rows_and_workspace_query(lib):
    assert _gemm(lib, M=0) == frt.FRT_OK
    assert frt.frt_packed_gemm_fp8_workspace_size(0, 768, 512) == 0
    need = frt.frt_packed_gemm_fp8_workspace_size(16, 768, 512)
    assert need >= 0
    if need:
        # a too-small workspace is refused before anything is launched
        assert _gemm(lib, ws_bytes=need - 1) == frt.FRT_E_INVALID
        assert "workspace" in frt.frt_last_error()
        assert _gemm(lib, ws=None, ws_bytes=0) == frt.FRT_E_INVALID
    # the default plans need no workspace
    for shape in [(2048, 32768, 16384), (4096, 9216, 3072), (64, 6144, 4096)]:
        assert frt.frt_packed_gemm_fp8_workspace_size(*shape) == 0


def test_pack_refusals(lib):
    def call(n_sib=2, Ns=(64, 32), K=128, Ws=(FAKE, FAKE + MB), Bs=None,
             W8=FAKE + 10 * MB, ws=FAKE + 11 * MB, bc=None):
        n = max(n_sib, 1)
        return lib.frt_pack_weights_fp8(
            None, n_sib, (ctypes.c_int64 * n)(*Ns[:n]), K,
            (ctypes.c_void_p * n)(*Ws[:n]),
            None if Bs is None else (ctypes.c_void_p * n)(*Bs), W8, ws, bc)
    assert call(n_sib=0) == frt.FRT_E_INVALID
    assert call(n_sib=17, Ns=[1] * 17, Ws=[FAKE] * 17) == frt.FRT_E_INVALID
    assert call(Ns=(64, 0)) == frt.FRT_E_INVALID
    assert call(K=0) == frt.FRT_E_INVALID
    assert call(Ws=(FAKE, None)) == frt.FRT_E_INVALID
    assert call(W8=FAKE + 100) == frt.FRT_E_INVALID     # over sibling 0
    assert "overlaps" in frt.frt_last_error()


def test_gemm_same_stride_overlap_is_exact(lib):
    """Splits written into one buffer with a shared row stride: columns
    that collide are refused (the interleaved, disjoint case is exercised
    on the GPU)."""
    o = FAKE + 40 * MB
    lds = [768, 768, 768]
    assert _gemm(lib, outs=[o, o + 500 * 2, o + 640 * 2], lds=lds) == frt.FRT_E_INVALID
    assert _gemm(lib, outs=[o + 600 * 2, o, o + 2 * MB], lds=lds) == frt.FRT_E_INVALID


def _geglu(lib, M=4, H=512, **kw):
    a = dict(stream=None, M=M, H=H, gu=FAKE, ld_gu=2 * H,
             act_scale=FAKE + 10 * MB, out_fp8=FAKE + 11 * MB, ld_out=H,
             y_f32=None, ld_y=0, amax_out=None)
    a.update(kw)
    return lib.frt_geglu_quant_fp8(*a.values())


def test_geglu_refusals(lib):
    assert _geglu(lib, H=0) == frt.FRT_E_INVALID
    assert _geglu(lib, M=-1) == frt.FRT_E_INVALID
    assert _geglu(lib, gu=None) == frt.FRT_E_INVALID
    assert _geglu(lib, ld_gu=1000) == frt.FRT_E_INVALID
    assert "ld_gu" in frt.frt_last_error()
    assert _geglu(lib, act_scale=None) == frt.FRT_E_INVALID
    assert _geglu(lib, ld_out=100) == frt.FRT_E_INVALID
    assert _geglu(lib, out_fp8=None) == frt.FRT_E_INVALID      # no output
    assert _geglu(lib, gu=FAKE + 1) == frt.FRT_E_INVALID        # misaligned
    assert _geglu(lib, out_fp8=FAKE + 512) == frt.FRT_E_INVALID  # over gu
    assert "overlaps" in frt.frt_last_error()
    assert _geglu(lib, y_f32=FAKE + 11 * MB + 256, ld_y=512) == frt.FRT_E_INVALID
    assert _geglu(lib, M=0) == frt.FRT_OK
    # odd H and unaligned strides are legal (the element-wise path)
    assert _geglu(lib, M=0, H=1001, ld_gu=2003, ld_out=1001) == frt.FRT_OK


def _gemm_geglu(lib, M=16, K=512, H=256, **kw):
    a = dict(stream=None, M=M, K=K, x8=FAKE, ld_x=K, W8=FAKE + MB, H=H,
             act_scale=FAKE + 30 * MB, w_scale=FAKE + 31 * MB, bias=None,
             out_scale=FAKE + 32 * MB, out_fp8=FAKE + 40 * MB, ld_out=H)
    a.update(kw)
    return lib.frt_packed_gemm_fp8_geglu_quant(*a.values())


def test_gemm_geglu_refusals(lib):
    assert _gemm_geglu(lib, K=256) == frt.FRT_E_INVALID
    assert _gemm_geglu(lib, K=520) == frt.FRT_E_UNSUPPORTED
    assert _gemm_geglu(lib, H=0) == frt.FRT_E_INVALID
    assert _gemm_geglu(lib, out_scale=None) == frt.FRT_E_INVALID
    assert _gemm_geglu(lib, out_fp8=None) == frt.FRT_E_INVALID
    assert _gemm_geglu(lib, ld_out=100) == frt.FRT_E_INVALID
    assert _gemm_geglu(lib, ld_x=520) == frt.FRT_E_INVALID
    assert _gemm_geglu(lib, W8=FAKE + MB + 8) == frt.FRT_E_INVALID
    # the codes over the packed weight (2H rows)
    assert _gemm_geglu(lib, out_fp8=FAKE + MB + 2 * 256 * 512 - 64) == frt.FRT_E_INVALID
    assert "overlaps" in frt.frt_last_error()
    assert _gemm_geglu(lib, M=0) == frt.FRT_OK


def test_interleave_refusals(lib):
    f = lib.frt_interleave_pairs_bf16
    assert f(None, 2, 7, 64, FAKE, FAKE + MB) == frt.FRT_E_INVALID      # odd hd
    assert f(None, 0, 8, 64, FAKE, FAKE + MB) == frt.FRT_E_INVALID
    assert f(None, 2, 8, 0, FAKE, FAKE + MB) == frt.FRT_E_INVALID
    assert f(None, 2, 8, 64, FAKE, None) == frt.FRT_E_INVALID
    assert f(None, 2, 8, 64, FAKE, FAKE + 64) == frt.FRT_E_INVALID       # overlap
    assert "overlaps" in frt.frt_last_error()


def _rope(lib, S=4, nh=2, kv=1, hd=64, P=8, T=16, **kw):
    a = dict(stream=None, S=S, nh=nh, kv=kv, hd=hd, qkv=FAKE, ld_qkv=(nh + 2 * kv) * hd,
             rope=FAKE + MB, P=P, T=T, q_out=FAKE + 2 * MB, k_cache=FAKE + 3 * MB,
             v_cache=FAKE + 4 * MB)
    a.update(kw)
    return lib.frt_qkv_split_rope_kvcache(*a.values())


def test_rope_split_refusals(lib):
    assert _rope(lib, hd=63) == frt.FRT_E_INVALID
    assert _rope(lib, kv=0) == frt.FRT_E_INVALID
    assert _rope(lib, P=13) == frt.FRT_E_INVALID          # P + S > T
    assert "cache rows" in frt.frt_last_error()
    assert _rope(lib, ld_qkv=100) == frt.FRT_E_INVALID
    assert _rope(lib, rope=None) == frt.FRT_E_INVALID
    assert _rope(lib, rope=FAKE + MB + 2) == frt.FRT_E_INVALID   # 4-byte rope
    # the written k rows over the v cache's written rows
    assert _rope(lib, v_cache=FAKE + 3 * MB) == frt.FRT_E_INVALID
    assert _rope(lib, q_out=FAKE + 64) == frt.FRT_E_INVALID       # over qkv
    assert _rope(lib, S=0) == frt.FRT_OK


def test_gemm_rope_refusals(lib):
    def call(**kw):
        a = dict(stream=None, M=16, K=512, x8=FAKE, ld_x=512, W8=FAKE + MB, nh=2, kv=1, hd=64,
                 act_scale=FAKE + 30 * MB, w_scale=FAKE + 31 * MB, bias=None,
                 rope=FAKE + 32 * MB, P=0, T=16, q_out=FAKE + 40 * MB,
                 k_cache=FAKE + 41 * MB, v_cache=FAKE + 42 * MB)
        a.update(kw)
        return lib.frt_packed_gemm_fp8_qkv_rope(*a.values())
    assert call(K=520) == frt.FRT_E_UNSUPPORTED
    assert call(hd=3) == frt.FRT_E_INVALID
    assert call(T=15) == frt.FRT_E_INVALID
    assert call(q_out=FAKE + MB) == frt.FRT_E_INVALID      # over W8
    assert call(w_scale=None) == frt.FRT_E_INVALID
    assert call(M=0) == frt.FRT_OK


def test_quantize_refusals(lib):
    f = lib.frt_quantize_fp8_static
    assert f(None, 4, 0, FAKE, 8, FAKE + MB, FAKE + 2 * MB, 8, None) == frt.FRT_E_INVALID
    assert f(None, 4, 512, FAKE, 500, FAKE + MB, FAKE + 2 * MB, 512, None) == frt.FRT_E_INVALID
    assert f(None, 4, 512, FAKE, 512, None, FAKE + 2 * MB, 512, None) == frt.FRT_E_INVALID
    assert f(None, 4, 512, FAKE, 512, FAKE + MB, None, 0, None) == frt.FRT_E_INVALID
    assert f(None, 4, 512, FAKE, 512, FAKE + MB, FAKE + 100, 512, None) == frt.FRT_E_INVALID
    assert "overlaps" in frt.frt_last_error()
    assert f(None, 0, 512, FAKE, 512, FAKE + MB, FAKE + 2 * MB, 512, None) == frt.FRT_OK


def test_gemm_bf16in_refusals(lib):
    def call(M=16, K=512, x=FAKE + 200 * MB, ld_x=512, x8=FAKE, ld_x8=512, **kw):
        splits = (768,)
        a = dict(stream=None, M=M, K=K, x=x, ld_x=ld_x, x8=x8, ld_x8=ld_x8, W8=FAKE + MB, N=768,
                 act_scale=FAKE + 30 * MB, w_scale=FAKE + 31 * MB, bias=None, n_split=1,
                 split_n=(ctypes.c_int64 * 1)(*splits), out=(ctypes.c_void_p * 1)(FAKE + 40 * MB),
                 ld_out=(ctypes.c_int64 * 1)(768), out_dtype=0, ws=None, ws_bytes=0)
        a.update(kw)
        return lib.frt_packed_gemm_bf16in_split(*a.values())
    assert call(x=None) == frt.FRT_E_INVALID
    assert call(ld_x=100) == frt.FRT_E_INVALID
    assert call(ld_x8=520) == frt.FRT_E_INVALID                   # the GEMM's x8 contract
    assert call(x8=FAKE + 200 * MB + 64) == frt.FRT_E_INVALID     # x8 over x
    assert call(x8=FAKE + MB) == frt.FRT_E_INVALID                # x8 over W8
    assert call(x=FAKE + 40 * MB) == frt.FRT_E_INVALID            # output over x
    assert call(M=0) == frt.FRT_OK


def test_mxfp4_refusals(lib):
    def pack(K=512, W=FAKE, W4=FAKE + 10 * MB, S4=FAKE + 11 * MB):
        return lib.frt_pack_weights_mxfp4(None, 1, (ctypes.c_int64 * 1)(64), K,
                                          (ctypes.c_void_p * 1)(W), None, W4, S4, None)
    assert pack(K=640) == frt.FRT_E_INVALID            # not a multiple of 256
    assert pack(W=FAKE + 8) == frt.FRT_E_INVALID       # 16-byte weights
    assert pack(S4=FAKE + 10 * MB + 100) == frt.FRT_E_INVALID   # S4 over W4
    assert "overlap" in frt.frt_last_error()

    def norm(D=512, **kw):
        a = dict(stream=None, M=4, D=D, residual=FAKE, ld_res=D, x=None, ld_x=0, gate=None, ld_gate=0,
                 weight=None, mod=FAKE + MB, ld_mod=0, eps=1e-6, residual_out=None, ld_rout=0,
                 out_fp4=FAKE + 2 * MB, ld_out=D // 2, out_scale=FAKE + 3 * MB, ld_sc=8 * 4,
                 gate_out=None, ld_gout=0)
        a.update(kw)
        return lib.frt_ada_norm_quant_mxfp4(*a.values())
    assert norm(D=640) == frt.FRT_E_INVALID               # D % 256
    assert norm(ld_out=200) == frt.FRT_E_INVALID
    assert norm(out_scale=None) == frt.FRT_E_INVALID
    assert norm(out_fp4=FAKE + 64) == frt.FRT_E_INVALID   # over residual
    assert norm(M=0) == frt.FRT_OK

    def gemm(K=512, **kw):
        a = dict(stream=None, M=16, K=K, x4=FAKE, ld_x4=K // 2, xs=FAKE + MB, ld_xs=8 * 16,
                 W4=FAKE + 2 * MB, S4=FAKE + 3 * MB, N=768, bias=None, n_split=1,
                 split_n=(ctypes.c_int64 * 1)(768), out=(ctypes.c_void_p * 1)(FAKE + 40 * MB),
                 ld_out=(ctypes.c_int64 * 1)(768), out_dtype=0)
        a.update(kw)
        return lib.frt_packed_gemm_mxfp4_split(*a.values())
    assert gemm(K=1000) == frt.FRT_E_INVALID
    assert gemm(K=640) == frt.FRT_E_INVALID               # K % 256
    assert gemm(ld_x4=200) == frt.FRT_E_INVALID
    assert gemm(xs=None) == frt.FRT_E_INVALID
    assert gemm(ld_xs=100) == frt.FRT_E_INVALID           # run stride < 8*M
    assert gemm(out=(ctypes.c_void_p * 1)(FAKE + 3 * MB)) == frt.FRT_E_INVALID   # over S4
    assert gemm(M=0) == frt.FRT_OK

    def geglu(K=512, **kw):
        a = dict(stream=None, M=16, K=K, x4=FAKE, ld_x4=K // 2, xs=FAKE + MB, ld_xs=8 * 16,
                 W4=FAKE + 2 * MB, S4=FAKE + 3 * MB, H=384, bias=None, out_scale=FAKE + 4 * MB,
                 out=FAKE + 40 * MB, ld_out=384)
        a.update(kw)
        return lib.frt_packed_gemm_mxfp4_geglu_quant(*a.values())
    assert geglu(K=640) == frt.FRT_E_INVALID              # K % 256
    assert geglu(H=0) == frt.FRT_E_INVALID
    assert geglu(xs=None) == frt.FRT_E_INVALID
    assert geglu(out_scale=None) == frt.FRT_E_INVALID
    assert geglu(ld_xs=100) == frt.FRT_E_INVALID          # run stride < 8*M
    assert geglu(ld_out=300) == frt.FRT_E_INVALID         # ld_out < H
    assert geglu(out=FAKE + 3 * MB) == frt.FRT_E_INVALID  # over S4
    assert geglu(M=0) == frt.FRT_OK

    def geglu4(K=512, **kw):
        a = dict(stream=None, M=16, K=K, x4=FAKE, ld_x4=K // 2, xs=FAKE + MB, ld_xs=8 * 16,
                 W4=FAKE + 2 * MB, S4=FAKE + 3 * MB, H=512, bias=None, out=FAKE + 40 * MB,
                 ld_out=256, sc=FAKE + 41 * MB, ld_sc=8 * 16)
        a.update(kw)
        return lib.frt_packed_gemm_mxfp4_geglu_mxfp4(*a.values())
    assert geglu4(H=384) == frt.FRT_E_INVALID              # H % 256
    assert geglu4(out=None) == frt.FRT_E_INVALID
    assert geglu4(sc=None) == frt.FRT_E_INVALID
    assert geglu4(ld_out=200) == frt.FRT_E_INVALID         # ld_out < H/2
    assert geglu4(ld_sc=100) == frt.FRT_E_INVALID          # run stride < 8*M
    assert geglu4(sc=FAKE + 40 * MB + 64) == frt.FRT_E_INVALID   # scales over the codes
    assert geglu4(M=0) == frt.FRT_OK

    def q4(fn, W=512, **kw):
        a = dict(stream=None, M=16, W=W, x=FAKE, ld_x=(2 if fn.endswith("geglu_quant_mxfp4") else 1) * W,
                 out=FAKE + 2 * MB, ld_out=W // 2, sc=FAKE + 3 * MB, ld_sc=8 * 16)
        a.update(kw)
        return getattr(lib, fn)(*a.values())
    for fn in ("frt_quantize_mxfp4", "frt_geglu_quant_mxfp4"):
        assert q4(fn, W=384) == frt.FRT_E_INVALID         # width % 256
        assert q4(fn, x=None) == frt.FRT_E_INVALID
        assert q4(fn, x=FAKE + 8) == frt.FRT_E_INVALID    # 16-byte input
        assert q4(fn, ld_out=200) == frt.FRT_E_INVALID    # ld_out < W/2
        assert q4(fn, ld_sc=100) == frt.FRT_E_INVALID     # run stride < 8*M
        assert q4(fn, out=FAKE + 64) == frt.FRT_E_INVALID  # over the input
        assert q4(fn, M=0) == frt.FRT_OK

    def mrope(K=512, **kw):
        a = dict(stream=None, M=16, K=K, x4=FAKE, ld_x4=K // 2, xs=FAKE + MB, ld_xs=8 * 16,
                 W4=FAKE + 2 * MB, S4=FAKE + 3 * MB, nh=4, kv=2, hd=64, bias=None,
                 rope=FAKE + 4 * MB, P=0, T=16, q=FAKE + 40 * MB, kc=FAKE + 41 * MB, vc=FAKE + 42 * MB)
        a.update(kw)
        return lib.frt_packed_gemm_mxfp4_qkv_rope(*a.values())
    assert mrope(K=640) == frt.FRT_E_INVALID              # K % 256
    assert mrope(xs=None) == frt.FRT_E_INVALID
    assert mrope(ld_xs=100) == frt.FRT_E_INVALID          # run stride < 8*M
    assert mrope(hd=63) == frt.FRT_E_INVALID              # odd head dim
    assert mrope(P=1) == frt.FRT_E_INVALID                # P + M > T
    assert mrope(q=FAKE + 3 * MB) == frt.FRT_E_INVALID    # q over S4
    assert mrope(M=0) == frt.FRT_OK


class _FakeDev:
    """Stands in for a device tensor in the binding's argument checks (its
    address is never dereferenced: the call below is refused first)."""

    def __init__(self, shape, dtype, addr):
        self.shape, self.dtype, self.is_cuda, self._addr = tuple(shape), dtype, True, addr
        self.device = "cuda:0"

    def data_ptr(self):
        return self._addr

    def dim(self):
        return len(self.shape)

    def stride(self, d=None):
        st = [1] * len(self.shape)
        for i in range(len(self.shape) - 2, -1, -1):
            st[i] = st[i + 1] * self.shape[i + 1]
        return tuple(st) if d is None else st[d]

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return 1


def test_binding_refuses_to_allocate_a_workspace(lib, monkeypatch):
    """A plan that needs a workspace is refused by the binding when the
    caller passes none: the binding never allocates one behind the call."""
    import torch
    monkeypatch.setattr(frt, "frt_packed_gemm_fp8_workspace_size", lambda M, N, K: 4096)
    x8 = _FakeDev((16, 512), torch.uint8, FAKE)
    W8 = _FakeDev((768, 512), torch.uint8, FAKE + MB)
    sc = _FakeDev((1,), torch.float32, FAKE + 2 * MB)
    out = _FakeDev((16, 768), torch.bfloat16, FAKE + 3 * MB)
    with pytest.raises(ValueError, match="workspace"):
        frt.frt_packed_gemm_fp8_split(x8, W8, sc, sc, [out], [768])
