// Device helpers shared by the frt HIP kernels (gfx950 / CDNA4).
//
// bf16 <-> fp32, the static FP8 e4m3fn quantiser, the tanh-form GELU and
// wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace frt {

constexpr float kFp8Max = 448.0f;  // largest finite e4m3fn magnitude

// bf16 halves of a 32-bit word (element 0 in the low half) -> fp32, exact.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  // NaN -> the sign and the quiet NaN 0x7fc0, selected by a mask (all ones
  // when |u| > 0x7f800000) rather than a branch
  const uint32_t nan = (uint32_t)((int32_t)(0x7f800000u - (u & 0x7fffffffu)) >> 31);
  return (r & ~nan) | ((((u >> 16) & 0x8000u) | 0x7fc0u) & nan);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// Correctly rounded y / s, given rcp = RN(1 / s) and s > 0 normal.
// q0 = y * rcp is within two ulps of y / s; one residual correction (the
// remainder y - q*s is exact under FMA for a near-quotient) brings it within
// half an ulp plus a tiny term, i.e. faithful; a second correction with the
// correctly rounded reciprocal then yields the correctly rounded quotient
// (Markstein's theorem on FMA-based division). Five VALU operations instead
// of the general division expansion. The corrections can turn a -0
// quotient into +0 (+0 + -0 = +0 under round-to-nearest); since s > 0 the
// quotient always carries y's sign, which copysign restores.
__device__ __forceinline__ float div_rn(float y, float s, float rcp) {
  float q = y * rcp;
  float r = __builtin_fmaf(-q, s, y);
  q = __builtin_fmaf(r, rcp, q);
  r = __builtin_fmaf(-q, s, y);
  return __builtin_copysignf(__builtin_fmaf(r, rcp, q), y);
}

// clamp to [-448, 448] keeping NaN (the definition's clamp propagates NaN).
__device__ __forceinline__ float clamp_fp8(float q) {
  float c = __builtin_amdgcn_fmed3f(q, -kFp8Max, kFp8Max);
  return (q != q) ? q : c;
}

// Four fp32 (already clamped) -> four e4m3fn codes in one dword, element 0
// in the low byte. v_cvt_pk_fp8_f32 rounds to nearest even (OCP e4m3fn on
// gfx950).
__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return uint32_t(w);
}
__device__ __forceinline__ uint32_t cvt2_fp8(float a, float b) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xffffu;
}

// Tanh-form GELU, 0.5 v (1 + tanh(z)) with z = sqrt(2/pi) (v + 0.044715 v^3),
// evaluated through the identity 0.5 (1 + tanh z) = 1 / (1 + e^(-2z)):
// gelu(v) = v / (1 + 2^(c v (1 + 0.044715 v^2))), c = -2 sqrt(2/pi) log2(e).
// No cancellation at either tail: for v -> -inf the power overflows to inf
// and the quotient is -0 (the tanh form's limit); for v -> +inf it is v.
__device__ __forceinline__ float gelu_tanh(float v) {
  constexpr float c = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  const float t = c * v * __builtin_fmaf(0.044715f, v * v, 1.0f);
  return v / (1.0f + __builtin_amdgcn_exp2f(t));
}

// ---- MXFP4 (OCP MX: e2m1 elements, one E8M0 scale per block of 32) ----

// e2m1 code of q (a value already divided by its block scale): nearest of
// 0, .5, 1, 1.5, 2, 3, 4, 6 with ties to the even code, saturating at 6;
// the sign bit is kept (bit 3).
__device__ __forceinline__ uint32_t e2m1_code(float q) {
  const float m = fabsf(q);
  const uint32_t idx = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                       (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
  return idx | ((__float_as_uint(q) >> 28) & 8u);
}

// E8M0 byte of a block from the fp32 bits of its max |v|: the OCP rule
// floor(log2(amax)) - 2, clamped at the bottom of the range (zero and
// subnormal maxima give byte 0); NaN or infinity give 0xFF.
__device__ __forceinline__ uint32_t e8m0_of_amax(uint32_t amax_bits) {
  const uint32_t e = (amax_bits >> 23) & 0xFFu;
  return e == 0xFFu ? 0xFFu : (e > 2u ? e - 2u : 0u);
}

// Eight values of one block -> eight e2m1 codes, element 0 in the low
// nibble; v / 2^(s - 127) is the exact power-of-two scaling ldexp.
__device__ __forceinline__ uint32_t mxfp4_pack8(const float* v, uint32_t sbyte) {
  const int sh = 127 - (int)sbyte;
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) w |= e2m1_code(__builtin_ldexpf(v[e], sh)) << (4 * e);
  return w;
}

// Byte offset of row m's block b in the MXFP4 scale layout: run-major
// [K/256][rows][8] with run stride ld_run, the 8 blocks of a run ordered
// 0, 2, 4, 6, 1, 3, 5, 7 (the order the GEMM's lanes consume them).
__device__ __forceinline__ int64_t e8m0_off(int64_t m, int64_t b, int64_t ld_run) {
  const int j = (int)(b & 7);
  return (b >> 3) * ld_run + m * 8 + ((j & 1) ? 4 + (j >> 1) : (j >> 1));
}

// Max of the four lanes of a quad (DPP xor 1, xor 2).
__device__ __forceinline__ uint32_t quad_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
  return v;
}

// The value held by lane l ^ 1 (DPP quad_perm [1,0,3,2]; the builtin is
// declared int-valued but moves the operand's bits, so the cast compiles
// to a plain DPP move).
__device__ __forceinline__ float lane_xor1(float v) {
  return static_cast<float>(__builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, true));
}

// ---- wave64 reductions (DPP within rows of 16, readlane across rows) ----

__device__ __forceinline__ float dpp_sum16(float v) {
  // quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2),
  // row_half_mirror (pairs the two quads of each 8-lane half),
  // row_mirror (pairs the two halves of each 16-lane row)
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, true);
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the 64 lanes; the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_sum16(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float dpp_max16(float v) {
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, true));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, true));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, true));
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, true));
  return v;
}

// Max over the 64 lanes of non-negative values (NaN-propagating through
// the unsigned bit order: NaN bit patterns sort above +inf).
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace frt
