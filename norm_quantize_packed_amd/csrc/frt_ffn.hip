// GEGLU of the merged gate/up GEMM output + static per-tensor FP8 e4m3fn.
//
// flashrt-structures 0.2.0, impls/adarms_stack/fp8_chain.py: `_quantize`
// packs the FFN's gate and up projections as one matrix, gate rows first,
// so the merged GEMM output row holds gate in columns [0, H) and up in
// [H, 2H); `_band_elements` (`down_project`) then turns that bf16 buffer
// into the FP8 input of the down projection (the chain's bind admits only
// tanh-GELU FFNs). Per row m < M and column j < H:
//   y = gelu_tanh(gate[m, j]) * up[m, j]                     (fp32)
//   out[m, j] = e4m3_rne(clamp(fl32(y / act_scale), -448, 448))
//
// Layout: thread t of block (bx, by) owns the VEC-column vector
// v = bx * 256 + t of rows by, by + gridDim.y, ... ; each wave's loads of
// the gate and the up half cover 64 consecutive 16-byte vectors (VEC = 8).
// The same epilogue also runs inside the gate/up GEMM (frt_gemm.hip), which
// skips the bf16 round trip through HBM.
//
// mx_quant_kernel: the 4-bit band's quantisers from bf16 (fp8_chain.py
// `BANDS`: the `fp4` row's quantize-from-bf16 entry, for a GEMM input that no
// norm producer writes, such as the attention output before the O
// projection; the `fp4_full` row's GELU-mul that emits packed 4-bit codes
// for a 4-bit down projection), in the OCP MXFP4 format: per row, blocks of
// 32 columns, one E8M0 scale 2^(floor(log2 max|v|) - 2) per block and the
// e2m1 codes of v / scale (nearest, ties to even, saturating at 6), two per
// byte; scales run-major [H/256][rows][8] as the MXFP4 GEMM reads them.
//
// quant_kernel: the plain static quantiser of a bf16 tensor (fp8_chain.py
// `_band_elements`, `out_project`: `quantize_fp8_static_bf16` of the
// attention output before the O projection; impls/linear_proj/
// fp8_static.py: the quantize that precedes the FP8 GEMM when the input
// arrives in bf16).
#include "frt_device.h"
#include "frt_internal.h"

namespace frt {

namespace {

template <int VEC>
__global__ __launch_bounds__(256) void geglu_kernel(GegluArgs a) {
  const int nv = a.H / VEC;
  const int v = blockIdx.x * 256 + threadIdx.x;
  const bool ok = v < nv;
  float s = 1.0f, rcp = 1.0f;
  if (a.out != nullptr) {
    s = *a.act_scale;
    rcp = 1.0f / s;
  }
  float amax = 0.0f;
  for (int64_t m = blockIdx.y; m < a.M && ok; m += gridDim.y) {
    const uint16_t* row = a.gu + m * a.ld_gu;
    const int64_t c = (int64_t)v * VEC;
    float y[VEC];
    if constexpr (VEC == 8) {
      const uint4 g = *reinterpret_cast<const uint4*>(row + c);
      const uint4 u = *reinterpret_cast<const uint4*>(row + a.H + c);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = (e & 1) ? bf16hi(gw[e >> 1]) : bf16lo(gw[e >> 1]);
        const float uv = (e & 1) ? bf16hi(uw[e >> 1]) : bf16lo(uw[e >> 1]);
        y[e] = gelu_tanh(gv) * uv;
      }
    } else {
      y[0] = gelu_tanh(bf16f(row[c])) * bf16f(row[a.H + c]);
    }
    if (a.y != nullptr) {
      float* yp = a.y + m * a.ld_y + c;
      if constexpr (VEC == 8) {
        reinterpret_cast<float4*>(yp)[0] = make_float4(y[0], y[1], y[2], y[3]);
        reinterpret_cast<float4*>(yp)[1] = make_float4(y[4], y[5], y[6], y[7]);
      } else {
        yp[0] = y[0];
      }
    }
    if (a.amax != nullptr) {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        amax = __uint_as_float(max(__float_as_uint(amax), __float_as_uint(fabsf(y[e]))));
    }
    if (a.out != nullptr) {
      float q[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[e] = clamp_fp8(div_rn(y[e], s, rcp));
      uint8_t* op = a.out + m * a.ld_out + c;
      if constexpr (VEC == 8) {
        uint2 t;
        t.x = cvt4_fp8(q[0], q[1], q[2], q[3]);
        t.y = cvt4_fp8(q[4], q[5], q[6], q[7]);
        *reinterpret_cast<uint2*>(op) = t;
      } else {
        op[0] = (uint8_t)cvt2_fp8(q[0], 0.0f);
      }
    }
  }
  if (a.amax != nullptr) {
    const uint32_t u = wave_umax(__float_as_uint(amax));
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(a.amax), u);
  }
}

// Static per-tensor FP8 of a bf16 tensor (the producers minus their norm):
// out[m, j] = e4m3_rne(clamp(fl32(x[m, j] / act_scale), -448, 448)), the
// same layout as geglu_kernel (x in the gate slot, no up half).
template <int VEC>
__global__ __launch_bounds__(256) void quant_kernel(GegluArgs a) {
  const int nv = a.H / VEC;
  const int v = blockIdx.x * 256 + threadIdx.x;
  const bool ok = v < nv;
  float s = 1.0f, rcp = 1.0f;
  if (a.out != nullptr) {
    s = *a.act_scale;
    rcp = 1.0f / s;
  }
  float amax = 0.0f;
  for (int64_t m = blockIdx.y; m < a.M && ok; m += gridDim.y) {
    const uint16_t* row = a.gu + m * a.ld_gu;
    const int64_t c = (int64_t)v * VEC;
    float y[VEC];
    if constexpr (VEC == 8) {
      const uint4 g = *reinterpret_cast<const uint4*>(row + c);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (e & 1) ? bf16hi(gw[e >> 1]) : bf16lo(gw[e >> 1]);
    } else {
      y[0] = bf16f(row[c]);
    }
    if (a.amax != nullptr) {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        amax = __uint_as_float(max(__float_as_uint(amax), __float_as_uint(fabsf(y[e]))));
    }
    if (a.out != nullptr) {
      float q[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) q[e] = clamp_fp8(div_rn(y[e], s, rcp));
      uint8_t* op = a.out + m * a.ld_out + c;
      if constexpr (VEC == 8) {
        uint2 t;
        t.x = cvt4_fp8(q[0], q[1], q[2], q[3]);
        t.y = cvt4_fp8(q[4], q[5], q[6], q[7]);
        *reinterpret_cast<uint2*>(op) = t;
      } else {
        op[0] = (uint8_t)cvt2_fp8(q[0], 0.0f);
      }
    }
  }
  if (a.amax != nullptr) {
    const uint32_t u = wave_umax(__float_as_uint(amax));
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(a.amax), u);
  }
}

// One thread per 8 columns; the four lanes of a quad hold one 32-column
// block (H % 32 == 0, so a quad is either wholly inside the row or wholly
// past its end).
template <bool GLU>
__global__ __launch_bounds__(256) void mx_quant_kernel(GegluArgs a) {
  const int nv = a.H / 8;
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= nv) return;
  for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
    const uint16_t* row = a.gu + m * a.ld_gu;
    const int64_t c = (int64_t)v * 8;
    const uint4 g = *reinterpret_cast<const uint4*>(row + c);
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    float y[8];
    if constexpr (GLU) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + a.H + c);
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = (e & 1) ? bf16hi(gw[e >> 1]) : bf16lo(gw[e >> 1]);
        const float uv = (e & 1) ? bf16hi(uw[e >> 1]) : bf16lo(uw[e >> 1]);
        y[e] = gelu_tanh(gv) * uv;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (e & 1) ? bf16hi(gw[e >> 1]) : bf16lo(gw[e >> 1]);
    }
    uint32_t am = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(fabsf(y[e])));
    const uint32_t sbyte = e8m0_of_amax(quad_umax(am));
    *reinterpret_cast<uint32_t*>(a.out + m * a.ld_out + c / 2) = mxfp4_pack8(y, sbyte);
    if ((threadIdx.x & 3) == 0) a.sc[e8m0_off(m, c / 32, a.ld_sc)] = (uint8_t)sbyte;
  }
}

}  // namespace

hipError_t launch_mx_quant(const GegluArgs& a, bool glu, hipStream_t st) {
  const int64_t nv = a.H / 8;
  const dim3 grid((unsigned)((nv + 255) / 256), (unsigned)(a.M < 65535 ? a.M : 65535));
  if (glu)
    hipLaunchKernelGGL((mx_quant_kernel<true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((mx_quant_kernel<false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_quant(const GegluArgs& a, int vec, hipStream_t st) {
  const int64_t nv = a.H / vec;
  const dim3 grid((unsigned)((nv + 255) / 256), (unsigned)(a.M < 65535 ? a.M : 65535));
  if (vec == 8)
    hipLaunchKernelGGL((quant_kernel<8>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((quant_kernel<1>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_geglu(const GegluArgs& a, int vec, hipStream_t st) {
  const int64_t nv = a.H / vec;
  const dim3 grid((unsigned)((nv + 255) / 256), (unsigned)(a.M < 65535 ? a.M : 65535));
  if (vec == 8)
    hipLaunchKernelGGL((geglu_kernel<8>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((geglu_kernel<1>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace frt
