// Joint-scale FP8 packing of sibling projections (flashrt-structures 0.2.0,
// impls/qkv_pack/fp8_static.py `_pack_weights`).
//
// Four stream-ordered launches, no workspace:
//   1. prep   : w_scale <- +0 (it accumulates max|W| as float bits while
//               the call runs) and bias_cat <- concat(b_i or zeros)
//   pack_mx:    the MXFP4 form: per-row blocks of 32 along K, e2m1 codes and
//               E8M0 scales (OCP MX rule), see frt_device.h
//   2. amax   : per sibling, block max of |w| bits -> atomicMax on w_scale
//   3. cast   : per sibling, codes = e4m3(clamp(fl32(w / s))), with
//               s = max(fl32(amax / 448), 1e-8) derived from w_scale's bits
//   4. final  : w_scale <- s
// For non-negative floats the IEEE bit order equals the numeric order, so
// an unsigned max over bit patterns is the float max (NaN sorts above +inf,
// so a NaN weight propagates as the definition's max does).
#include "frt_device.h"
#include "frt_internal.h"

namespace frt {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float pack_scale_from_amax(uint32_t amax_bits) {
  const float s = __uint_as_float(amax_bits) / kFp8Max;  // correctly rounded
  return (s != s) ? s : fmaxf(s, 1e-8f);
}

__global__ __launch_bounds__(kThreads) void pack_prep_kernel(
    float* w_scale, uint16_t* bias_cat, const uint16_t* b, int64_t n, int64_t off, int first) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (first && t == 0) *reinterpret_cast<uint32_t*>(w_scale) = 0u;
  if (bias_cat != nullptr && t < n) bias_cat[off + t] = (b != nullptr) ? b[t] : (uint16_t)0;
}

// |bf16| bit patterns of a word's two halves, widened to fp32 bit order
__device__ __forceinline__ uint32_t absmax2(uint32_t w) {
  return max((w & 0x7fffu) << 16, w & 0x7fff0000u);
}

// Each thread folds 8 elements per load when the sibling is 16-byte aligned
// and a multiple of 8 long (four independent loads per step), else one
// element per step. The block's four wave maxima meet in LDS; one thread
// then raises w_scale, skipping the atomic when the agent-coherent value is
// already at least as large (most blocks, once the first ones have run).
template <bool V8>
__global__ __launch_bounds__(kThreads) void pack_amax_kernel(const uint16_t* w, int64_t elems,
                                                              float* w_scale) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  if constexpr (V8) {
    const uint4* w4 = reinterpret_cast<const uint4*>(w);
    const int64_t n4 = elems / 8;
    int64_t i = t0;
    for (; i + 3 * stride < n4; i += 4 * stride) {
      uint4 t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) t[u] = w4[i + u * stride];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        m = max(m, max(max(absmax2(t[u].x), absmax2(t[u].y)), max(absmax2(t[u].z), absmax2(t[u].w))));
    }
    for (; i < n4; i += stride) {
      const uint4 t = w4[i];
      m = max(m, max(max(absmax2(t.x), absmax2(t.y)), max(absmax2(t.z), absmax2(t.w))));
    }
  } else {
    for (int64_t i = t0; i < elems; i += stride) m = max(m, (uint32_t)(w[i] & 0x7fffu) << 16);
  }
  m = wave_umax(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) m = max(m, red[k]);
    unsigned int* p = reinterpret_cast<unsigned int*>(w_scale);
    if (m > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, m);
  }
}

template <bool V8>
__global__ __launch_bounds__(kThreads) void pack_cast_kernel(const uint16_t* w, int64_t elems,
                                                              uint8_t* dst, const float* w_scale) {
  const float s = pack_scale_from_amax(*reinterpret_cast<const uint32_t*>(w_scale));
  const float rcp = 1.0f / s;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if constexpr (V8) {
    const uint4* w4 = reinterpret_cast<const uint4*>(w);
    uint2* d2 = reinterpret_cast<uint2*>(dst);
    const int64_t n4 = elems / 8;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
      const uint4 t = w4[i];
      const uint32_t ws[4] = {t.x, t.y, t.z, t.w};
      float q[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q[2 * k] = clamp_fp8(div_rn(bf16lo(ws[k]), s, rcp));
        q[2 * k + 1] = clamp_fp8(div_rn(bf16hi(ws[k]), s, rcp));
      }
      uint2 o;
      o.x = cvt4_fp8(q[0], q[1], q[2], q[3]);
      o.y = cvt4_fp8(q[4], q[5], q[6], q[7]);
      d2[i] = o;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < elems; i += stride) {
      const float q = clamp_fp8(div_rn(bf16f(w[i]), s, rcp));
      dst[i] = (uint8_t)(cvt2_fp8(q, 0.0f) & 0xffu);
    }
  }
}

__global__ void pack_final_kernel(float* w_scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0)
    *w_scale = pack_scale_from_amax(*reinterpret_cast<const uint32_t*>(w_scale));
}

unsigned grid_for(int64_t work, int64_t cap = 4096) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g > cap) g = cap;  // grid-stride beyond the cap
  if (g < 1) g = 1;
  return (unsigned)g;
}

// MXFP4 pack of one sibling (K % 256 == 0): thread t takes 8 consecutive
// elements of a row (16-byte load), the four threads of a quad one block of
// 32; rows follow each other, so a quad never straddles a row. Threads past
// the end still take part in the quad max (with zeros) and store nothing.
// scales: the packed matrix's run-major scale array offset to this
// sibling's first row (run stride = 8 x all packed rows).
__global__ __launch_bounds__(kThreads) void pack_mx_kernel(const uint16_t* w, int64_t rows, int64_t K,
                                                           uint8_t* codes, uint8_t* scales, int64_t rows_total) {
  const int64_t nv = K / 8;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool ok = t < rows * nv;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int64_t row = ok ? t / nv : 0, vv = ok ? t - row * nv : 0;
  if (ok) {
    const uint4 q = *reinterpret_cast<const uint4*>(w + row * K + vv * 8);
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (e & 1) ? bf16hi(wd[e >> 1]) : bf16lo(wd[e >> 1]);
  }
  uint32_t am = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(fabsf(v[e])));
  const uint32_t sbyte = e8m0_of_amax(quad_umax(am));
  if (ok) {
    *reinterpret_cast<uint32_t*>(codes + row * (K / 2) + vv * 4) = mxfp4_pack8(v, sbyte);
    if ((threadIdx.x & 3) == 0) scales[e8m0_off(row, vv / 4, rows_total * 8)] = (uint8_t)sbyte;
  }
}

}  // namespace

hipError_t launch_pack_mxfp4(const PackSib* sibs, int n_sib, int64_t K, uint8_t* w4, uint8_t* s4,
                             uint16_t* bias_cat, hipStream_t st) {
  const int64_t rows_total = sibs[n_sib - 1].row_off + sibs[n_sib - 1].rows;
  for (int i = 0; i < n_sib; ++i) {
    if (bias_cat != nullptr)
      hipLaunchKernelGGL(pack_prep_kernel, dim3(grid_for(sibs[i].rows)), dim3(kThreads), 0, st, nullptr,
                         bias_cat, sibs[i].b, sibs[i].rows, sibs[i].row_off, 0);
    const int64_t threads = sibs[i].rows * (K / 8);
    hipLaunchKernelGGL(pack_mx_kernel, dim3((unsigned)((threads + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       st, sibs[i].w, sibs[i].rows, K, w4 + sibs[i].row_off * (K / 2), s4 + sibs[i].row_off * 8,
                       rows_total);
  }
  return hipGetLastError();
}

hipError_t launch_pack(const PackSib* sibs, int n_sib, int64_t K, uint8_t* w8, float* w_scale,
                       uint16_t* bias_cat, hipStream_t st) {
  (void)K;
  for (int i = 0; i < n_sib; ++i) {
    const int64_t n = bias_cat != nullptr ? sibs[i].rows : 1;
    hipLaunchKernelGGL(pack_prep_kernel, dim3(grid_for(n)), dim3(kThreads), 0, st, w_scale, bias_cat,
                       sibs[i].b, sibs[i].rows, sibs[i].row_off, i == 0 ? 1 : 0);
  }
  for (int i = 0; i < n_sib; ++i) {
    const PackSib& p = sibs[i];
    const bool v8 = (p.elems % 8 == 0) && ((uintptr_t)p.w % 16 == 0);
    if (v8)
      hipLaunchKernelGGL(pack_amax_kernel<true>, dim3(grid_for(p.elems / 8, 1024)), dim3(kThreads), 0, st,
                         p.w, p.elems, w_scale);
    else
      hipLaunchKernelGGL(pack_amax_kernel<false>, dim3(grid_for(p.elems, 1024)), dim3(kThreads), 0, st, p.w,
                         p.elems, w_scale);
  }
  for (int i = 0; i < n_sib; ++i) {
    const PackSib& p = sibs[i];
    uint8_t* dst = w8 + p.dst_off;
    const bool v8 = (p.elems % 8 == 0) && ((uintptr_t)p.w % 16 == 0) && ((uintptr_t)dst % 8 == 0);
    if (v8)
      hipLaunchKernelGGL(pack_cast_kernel<true>, dim3(grid_for(p.elems / 8)), dim3(kThreads), 0, st,
                         p.w, p.elems, dst, w_scale);
    else
      hipLaunchKernelGGL(pack_cast_kernel<false>, dim3(grid_for(p.elems)), dim3(kThreads), 0, st, p.w,
                         p.elems, dst, w_scale);
  }
  hipLaunchKernelGGL(pack_final_kernel, dim3(1), dim3(64), 0, st, w_scale);
  return hipGetLastError();
}

}  // namespace frt
