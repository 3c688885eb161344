// Internal kernel-argument structs and launchers of the frt library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/frt.h"

namespace frt {

struct AdaArgs {
  const uint16_t* res; int64_t ld_res;
  const uint16_t* x; int64_t ld_x;
  const uint16_t* gate; int64_t ld_gate;
  const uint16_t* weight;
  const uint16_t* mod; int64_t ld_mod;
  const float* act_scale; float eps;
  uint16_t* rout; int64_t ld_rout;
  uint8_t* out; int64_t ld_out;
  uint16_t* gout; int64_t ld_gout;
  float* y; int64_t ld_y;
  float* amax;
  int64_t M; int D;
  // MXFP4 output (launch_ada_norm_mxfp4): e2m1 codes in out ([M, ld_out]
  // bytes, two per byte) and E8M0 block scales in sc, run-major
  // [D/256][rows][8] with run stride ld_sc
  uint8_t* sc; int64_t ld_sc;
};

struct PtokArgs {
  const uint16_t* x; int64_t ld_x;
  const uint16_t* temb; int64_t ld_temb;
  const float* table;
  const float* act_scale; float eps;
  int shift_idx, scale_idx;
  uint8_t* out; int64_t ld_out;
  float* y; int64_t ld_y;
  float* amax;
  int64_t R; int D;
};

hipError_t launch_ada_norm(const AdaArgs& a, bool vec8, hipStream_t st);
hipError_t launch_ada_norm_mxfp4(const AdaArgs& a, hipStream_t st);
hipError_t launch_ptok_norm(const PtokArgs& a, bool vec8, hipStream_t st);

struct PackSib {
  const uint16_t* w;      // bf16 [n, K]
  const uint16_t* b;      // bf16 [n] or null
  int64_t elems;          // n * K
  int64_t dst_off;        // element offset of this sibling in W8
  int64_t rows, row_off;  // n, sum of earlier n
};

hipError_t launch_pack(const PackSib* sibs, int n_sib, int64_t K, uint8_t* w8,
                       float* w_scale, uint16_t* bias_cat, hipStream_t st);
// MXFP4 pack: codes [sum N, K/2], E8M0 scales run-major [K/256][sum N][8]
hipError_t launch_pack_mxfp4(const PackSib* sibs, int n_sib, int64_t K, uint8_t* w4, uint8_t* s4,
                             uint16_t* bias_cat, hipStream_t st);

struct SplitTab {
  void* ptr[FRT_MAX_SPLITS];
  int64_t ld[FRT_MAX_SPLITS];
  int off[FRT_MAX_SPLITS + 1];
  int n;
};

struct GemmArgs {
  const uint8_t* x; int64_t ld_x;
  const uint8_t* w;
  const float* act_scale; const float* w_scale;
  const uint16_t* bias;
  int M, N, K;
  int out_f32;
  SplitTab sp;
  // bf16 outputs whose split widths and row strides are multiples of 8
  // elements and whose pointers are 16-byte aligned: the 256-row plans then
  // store 16 bytes a lane
  int vec_out;
  // gate/up GEGLU epilogue (launch_gemm_geglu): W8 holds 2H rows, gate
  // first; codes of gelu_tanh(gate) * up go to q8 [M, ld_q8] at q_scale
  int H;
  uint8_t* q8; int64_t ld_q8;
  const float* q_scale;
  // QKV split + RoPE + KV-cache epilogue (launch_gemm_rope): N = (nh + 2kv)
  // hd columns q | k | v, q/k rows pair-interleaved; token m uses rope row
  // m, writes q_out row m and cache row P + m
  const uint16_t* rope;
  int nh, kv, hd;
  int64_t P;
  uint16_t* q_out; uint16_t* k_cache; uint16_t* v_cache;
  // MXFP4 operands (launch_gemm_mxfp4): x, w hold e2m1 codes (K/2 bytes a
  // row, ld_x in bytes); E8M0 block scales run-major [K/256][rows][8]: sa
  // with run stride ld_sa, sb with run stride 8 N
  const uint8_t* sa; int64_t ld_sa;
  const uint8_t* sb;
  // GEGLU form with an MXFP4 output (q4 non-null, instead of q8): codes
  // [M, ld_q4] two per byte, scales run-major [H/256][rows][8] with run
  // stride ld_sc4; H % 256 == 0
  uint8_t* q4; int64_t ld_q4;
  uint8_t* sc4; int64_t ld_sc4;
  // first output column of the tiles a launch covers (the 256-row split
  // plan's second launch of narrower tiles over the last columns; else 0)
  int n_base;
};

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
// compute units of the current device (cached per device)
int device_cus();
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_geglu(const GemmArgs& a, hipStream_t st);

struct GegluArgs {
  const uint16_t* gu; int64_t ld_gu;
  const float* act_scale;
  uint8_t* out; int64_t ld_out;
  float* y; int64_t ld_y;
  float* amax;
  int64_t M; int H;
  uint8_t* sc; int64_t ld_sc;   // MXFP4 block scales (launch_mx_quant)
};

hipError_t launch_geglu(const GegluArgs& a, int vec, hipStream_t st);
// static FP8 of a bf16 [M, H] tensor (GegluArgs with gu = x, no up half)
hipError_t launch_quant(const GegluArgs& a, int vec, hipStream_t st);
// MXFP4 of a bf16 [M, H] tensor (glu = false) or of the GEGLU of a bf16
// gate|up [M, 2H] buffer (glu = true): codes into out, scales into sc
hipError_t launch_mx_quant(const GegluArgs& a, bool glu, hipStream_t st);

hipError_t launch_gemm_rope(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mxfp4_geglu(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_mxfp4_rope(const GemmArgs& a, hipStream_t st);

struct RopeArgs {
  const uint16_t* qkv; int64_t ld_qkv;
  const uint16_t* rope;
  int nh, kv, hd;
  int64_t S, P;
  uint16_t* q_out; uint16_t* k_cache; uint16_t* v_cache;
};

hipError_t launch_rope_split(const RopeArgs& a, int vec, hipStream_t st);
hipError_t launch_interleave(const uint16_t* src, uint16_t* dst, int nheads, int hd, int64_t K, int vec,
                             hipStream_t st);

}  // namespace frt
