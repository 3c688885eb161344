"""CPU oracle for the norm-quantize producers and the packed FP8 GEMM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import or call this package; only the tests, the
entry point's smoke check and the bench's CPU-baseline leg do.

It is a plain, slow, obviously-correct NumPy implementation of what the
pages compute, written from their definitions (flashrt-structures 0.2.0
wheel pages): fp64 arithmetic wherever the pages do not fix the precision,
exact integer arithmetic for the FP8 GEMM, and the codecs (bf16, e4m3fn)
written out from the formats' definitions. It shares no code with the HIP
path. Each function names the passage it follows.

Modules:
  codecs     bf16 and e4m3fn encode/decode, signed code ordinals
  producers  gated residual + AdaRMS, per-token-table LayerNorm, static
             per-tensor FP8 quantisation, calibration scale
  pack       joint-scale sibling weight packing
  gemm       exact packed FP8 GEMM, dequant + bias epilogue, column split
  ffn        tanh-GELU GEGLU of the merged gate/up output + static FP8,
             and the merged gate/up GEMM -> GEGLU chain
  rope       q/k pair interleave, QKV split + adjacent-pair RoPE + KV-cache
             write
  mxfp4      OCP MX FP4 codec, block quantiser, block-scaled GEMM

Parity status: every function is pinned by the ``-m "not gpu"`` tests in
tests/test_oracle_*.py (closed forms, brute force, independent torch CPU
routines). None is "parity unpinned".
"""

from .codecs import (bf16_to_f32, f32_to_bf16, e4m3_decode, e4m3_encode,
                     e4m3_ordinal, e4m3_int, E4M3_MAX)
from .producers import (gated_residual, ada_rms_norm, ada_norm_quant_fp8,
                        ptok_layer_norm, ptok_norm_quant_fp8,
                        quantize_static, calibrate_act_scale)
from .pack import pack_weights
from .gemm import (gemm_exact, gemm_exact_at, epilogue, packed_gemm_split,
                   split_columns)
from .ffn import gelu_tanh, geglu, geglu_quant_fp8, gate_up_gelu_quant
from .rope import pair_perm, interleave_rows, rotate_pairs, qkv_split_rope_kvcache
from . import mxfp4

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "e4m3_decode", "e4m3_encode",
    "e4m3_ordinal", "e4m3_int", "E4M3_MAX",
    "gated_residual", "ada_rms_norm", "ada_norm_quant_fp8",
    "ptok_layer_norm", "ptok_norm_quant_fp8", "quantize_static",
    "calibrate_act_scale", "pack_weights", "gemm_exact", "gemm_exact_at",
    "epilogue", "packed_gemm_split", "split_columns",
    "gelu_tanh", "geglu", "geglu_quant_fp8", "gate_up_gelu_quant",
    "pair_perm", "interleave_rows", "rotate_pairs", "qkv_split_rope_kvcache",
]
