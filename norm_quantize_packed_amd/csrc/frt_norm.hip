// Conditioned-norm producers with static per-tensor FP8 e4m3fn output.
//
//  - ada_norm_kernel: gated residual + AdaRMS (flashrt-structures 0.2.0,
//    impls/adarms_stack/fp8_chain.py: the fused producer of `_band_elements`,
//    the arithmetic of the stack tail in `_make_run`).
//  - ptok_norm_kernel: per-token-table no-affine adaptive LayerNorm
//    (impls/modnorm_qkv_chain/fp8_ptok_table.py, module docstring and
//    `PerTokenModChainBlock.forward`).
//
// Layout: one row is owned by WPR wavefronts: WPR = 1, 2 or 4 waves of a
// 256-thread block holding 4 / WPR rows, or WPR = 8 waves of a 512-thread
// block holding one row (short calls spread over more CUs). Lane `l` of the row's
// wave `w` handles the VEC-element vectors v = w*64 + l + i*64*WPR,
// i < NV, so each load instruction of a wave covers 64 consecutive vectors
// (fully coalesced 16-byte accesses on the VEC = 8 path). The row stays in
// registers between the statistics pass and the output pass, so every input
// byte is read from HBM once. Row statistics are reduced with DPP inside
// rows of 16 lanes, readlane across the four rows of the wave, and LDS
// across the WPR waves of a row.
#include "frt_device.h"
#include "frt_internal.h"

namespace frt {

namespace {

template <int VEC>
struct Vec;
template <>
struct Vec<8> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const uint16_t* p) {
    uint4 t = *reinterpret_cast<const uint4*>(p);
    w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
  }
  // non-temporal: for inputs this launch reads exactly once (a hit is still
  // served from the caches; a miss allocates nothing there)
  __device__ __forceinline__ void load_once(const uint16_t* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
  }
  __device__ __forceinline__ void store(uint16_t* p) const {
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ __forceinline__ float f(int e) const { return (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]); }
};
template <>
struct Vec<2> {
  uint32_t w[1];
  __device__ __forceinline__ void load(const uint16_t* p) { w[0] = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void load_once(const uint16_t* p) { load(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint32_t*>(p) = w[0]; }
  __device__ __forceinline__ float f(int e) const { return e ? bf16hi(w[0]) : bf16lo(w[0]); }
};

template <int VEC>
__device__ __forceinline__ void store_codes(uint8_t* p, const float* q);
template <>
__device__ __forceinline__ void store_codes<8>(uint8_t* p, const float* q) {
  uint2 t;
  t.x = cvt4_fp8(q[0], q[1], q[2], q[3]);
  t.y = cvt4_fp8(q[4], q[5], q[6], q[7]);
  *reinterpret_cast<uint2*>(p) = t;
}
template <>
__device__ __forceinline__ void store_codes<2>(uint8_t* p, const float* q) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)cvt2_fp8(q[0], q[1]);
}

template <int VEC>
__device__ __forceinline__ void store_f32(float* p, const float* v) {
  if constexpr (VEC == 8) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
}

template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float* v) {
  if constexpr (VEC == 8) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    float2 a = *reinterpret_cast<const float2*>(p);
    v[0] = a.x; v[1] = a.y;
  }
}

// Sum of `v` over the WPR waves that own this row (wave-uniform result).
// Every thread of the block must call it (it contains a barrier when
// WPR > 1).
template <int WPR>
__device__ __forceinline__ float row_sum(float v, float* red, int wave) {
  float s = wave_sum(v);
  if constexpr (WPR == 1) {
    return s;
  } else {
    __syncthreads();  // previous use of `red` finished
    if ((threadIdx.x & 63) == 0) red[wave] = s;
    __syncthreads();
    const int base = wave - wave % WPR;  // first wave of this row
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < WPR; ++k) t += red[base + k];
    return t;
  }
}

__device__ __forceinline__ void amax_commit(float* amax, float m) {
  uint32_t u = wave_umax(__float_as_uint(m));
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int*>(amax), u);
}

}  // namespace

// MX: MXFP4 output instead of static FP8 (vector path, D % 256 == 0): the
// four lanes of a quad hold 32 consecutive columns, one block; its max
// comes from two DPP steps, then each lane writes its 8 codes (4 bytes) and
// the quad's first lane the block's scale byte (run-major layout, run
// stride ld_sc).
template <int WPR, int NV, int VEC, bool MX = false>
__global__ __launch_bounds__(WPR <= 4 ? 256 : 64 * WPR) void ada_norm_kernel(AdaArgs a) {
  constexpr int RPB = WPR <= 4 ? 4 / WPR : 1;
  constexpr bool EARLY = NV <= 4;  // modulation loads issued before the reduction
  __shared__ float red[WPR <= 4 ? 4 : WPR];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
  const int sub = wave % WPR;
  const bool row_ok = row < a.M;
  const int nvec = a.D / VEC;
  const uint16_t* mrow = a.mod + row * a.ld_mod;

  float h[NV][VEC];
  Vec<VEC> msc[EARLY ? NV : 1], msh[EARLY ? NV : 1], mw[EARLY ? NV : 1], mg[EARLY ? NV : 1];
  // the quantiser scale (and, with EARLY, the gate chunk echoed to gate_out)
  // is read with the row's first loads: read after the reduction's barrier,
  // its latency trailed the row (with one block per row and few rows, a
  // visible tail: 16 x 512 2.65 -> 2.53 us; level at 64 x 4096 and 256 x
  // 2048)
  float s = 1.0f;
  if (!MX && a.out != nullptr) s = *a.act_scale;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = sub * 64 + lane + i * 64 * WPR;
    if (row_ok && v < nvec) {
      const int64_t c = (int64_t)v * VEC;
      Vec<VEC> r;
      r.load(a.res + row * a.ld_res + c);
      if constexpr (EARLY) {
        msc[i].load(mrow + c);
        msh[i].load(mrow + a.D + c);
        if (a.weight != nullptr) mw[i].load(a.weight + c);
        if (a.gout != nullptr) mg[i].load(mrow + 2 * a.D + c);
      }
      if (a.x != nullptr && a.gate != nullptr) {
        Vec<VEC> x, g;
        x.load(a.x + row * a.ld_x + c);
        g.load(a.gate + row * a.ld_gate + c);  // ld_gate == 0: broadcast row
#pragma unroll
        for (int e = 0; e < VEC; ++e) h[i][e] = __builtin_fmaf(g.f(e), x.f(e), r.f(e));
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) h[i][e] = r.f(e);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss = __builtin_fmaf(h[i][e], h[i][e], ss);
      if (a.rout != nullptr) {
        Vec<VEC> o;
#pragma unroll
        for (int e = 0; e < VEC; e += 2) o.w[e >> 1] = pack_bf2(h[i][e], h[i][e + 1]);
        o.store(a.rout + row * a.ld_rout + c);
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) h[i][e] = 0.0f;
    }
  }
  const float tot = row_sum<WPR>(ss, red, wave);
  const float rr = __builtin_amdgcn_rsqf(tot / (float)a.D + a.eps);

  const float rcp = 1.0f / s;
  float amax = 0.0f;
  if (row_ok) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = sub * 64 + lane + i * 64 * WPR;
      if (v < nvec) {
        const int64_t c = (int64_t)v * VEC;
        Vec<VEC> sc, sh, w;
        if constexpr (EARLY) {
          sc = msc[i];
          sh = msh[i];
          w = mw[i];
        } else {
          sc.load(mrow + c);
          sh.load(mrow + a.D + c);
          if (a.weight != nullptr) w.load(a.weight + c);
        }
        float y[VEC];
        if (a.weight != nullptr) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) y[e] = h[i][e] * rr * w.f(e);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) y[e] = h[i][e] * rr;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] = __builtin_fmaf(y[e], sc.f(e), y[e]) + sh.f(e);
        if (a.y != nullptr) store_f32<VEC>(a.y + row * a.ld_y + c, y);
        if (a.amax != nullptr) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) amax = __uint_as_float(max(__float_as_uint(amax), __float_as_uint(fabsf(y[e]))));
        }
        if constexpr (MX) {
          static_assert(!MX || VEC == 8, "MXFP4 output takes the vector path");
          uint32_t am = 0;
#pragma unroll
          for (int e = 0; e < VEC; ++e) am = max(am, __float_as_uint(fabsf(y[e])));
          const uint32_t sbyte = e8m0_of_amax(quad_umax(am));
          *reinterpret_cast<uint32_t*>(a.out + row * a.ld_out + c / 2) = mxfp4_pack8(y, sbyte);
          if ((lane & 3) == 0) a.sc[e8m0_off(row, c / 32, a.ld_sc)] = (uint8_t)sbyte;
        } else if (a.out != nullptr) {
          float q[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) q[e] = clamp_fp8(div_rn(y[e], s, rcp));
          store_codes<VEC>(a.out + row * a.ld_out + c, q);
        }
        if (a.gout != nullptr) {
          Vec<VEC> g;
          if constexpr (EARLY)
            g = mg[i];
          else
            g.load(mrow + 2 * a.D + c);
          g.store(a.gout + row * a.ld_gout + c);
        }
      }
    }
  }
  if (a.amax != nullptr) amax_commit(a.amax, amax);
}

template <int WPR, int NV, int VEC>
__global__ __launch_bounds__(WPR <= 4 ? 256 : 64 * WPR) void ptok_norm_kernel(PtokArgs a) {
  constexpr int RPB = WPR <= 4 ? 4 / WPR : 1;
  // table loads issued before the reductions while the registers allow it
  // (at 4 vectors per lane the extra 64 registers cost more occupancy than
  // the early loads save)
  constexpr bool EARLY = NV <= 3;
  __shared__ float red[WPR <= 4 ? 4 : WPR];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
  const int sub = wave % WPR;
  const bool row_ok = row < a.R;
  const int nvec = a.D / VEC;
  const float* tab_s = a.table + (int64_t)a.shift_idx * a.D;
  const float* tab_c = a.table + (int64_t)a.scale_idx * a.D;

  // x stays in its packed bf16 form (16 bytes a vector) and is widened
  // where it is used, which keeps more rows in flight per CU
  Vec<VEC> xv[NV];
  Vec<VEC> tsh[NV], tsc[NV];
  float ts[EARLY ? NV : 1][VEC], tc[EARLY ? NV : 1][VEC];
  float sum = 0.0f;
  const uint16_t* trow = a.temb + row * a.ld_temb;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = sub * 64 + lane + i * 64 * WPR;
    if (row_ok && v < nvec) {
      const int64_t c = (int64_t)v * VEC;
      // x and the two temb chunks are read once (inputs rotated past the
      // caches, 2048 x 16384: 53.3 -> 50.9 us; 8192 x 3072: 39.5 -> 38.2);
      // the table rows, read by every row, keep the default policy
      xv[i].load_once(a.x + row * a.ld_x + c);
      tsh[i].load_once(trow + (int64_t)a.shift_idx * a.D + c);
      tsc[i].load_once(trow + (int64_t)a.scale_idx * a.D + c);
      if constexpr (EARLY) {
        load_f32<VEC>(tab_s + c, ts[i]);
        load_f32<VEC>(tab_c + c, tc[i]);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) sum += xv[i].f(e);
    }
  }
  const float inv_d = 1.0f / (float)a.D;
  const float mu = row_sum<WPR>(sum, red, wave) * inv_d;
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = sub * 64 + lane + i * 64 * WPR;
    if (row_ok && v < nvec) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = xv[i].f(e) - mu;
        sq = __builtin_fmaf(d, d, sq);
      }
    }
  }
  const float var = row_sum<WPR>(sq, red, wave) * inv_d;
  const float rstd = __builtin_amdgcn_rsqf(var + a.eps);

  // (the quantiser scale read here, after the reductions: read with the
  // row's first loads it measured slower, 8192 x 3072: 35.9 -> 36.7 us)
  float s = 1.0f, rcp = 1.0f;
  if (a.out != nullptr) {
    s = *a.act_scale;
    rcp = 1.0f / s;
  }
  float amax = 0.0f;
  if (row_ok) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = sub * 64 + lane + i * 64 * WPR;
      if (v < nvec) {
        const int64_t c = (int64_t)v * VEC;
        float tsv[VEC], tcv[VEC], y[VEC];
        if constexpr (EARLY) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            tsv[e] = ts[i][e];
            tcv[e] = tc[i][e];
          }
        } else {
          load_f32<VEC>(tab_s + c, tsv);
          load_f32<VEC>(tab_c + c, tcv);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float shift = tsv[e] + tsh[i].f(e);
          const float scale = tcv[e] + tsc[i].f(e);
          const float n = (xv[i].f(e) - mu) * rstd;
          y[e] = __builtin_fmaf(n, scale, n) + shift;
        }
        if (a.y != nullptr) store_f32<VEC>(a.y + row * a.ld_y + c, y);
        if (a.amax != nullptr) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) amax = __uint_as_float(max(__float_as_uint(amax), __float_as_uint(fabsf(y[e]))));
        }
        if (a.out != nullptr) {
          float q[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) q[e] = clamp_fp8(div_rn(y[e], s, rcp));
          store_codes<VEC>(a.out + row * a.ld_out + c, q);
        }
      }
    }
  }
  if (a.amax != nullptr) amax_commit(a.amax, amax);
}

// ---------------------------------------------------------------- launchers

namespace {

// Waves per row: at most 32 elements per lane on the vector path (keeps
// the row, its modulation and the statistics in registers at a useful
// occupancy), and more waves when rows are scarce so that short calls still
// spread across the chip. 8 waves per row use 512-thread blocks.
int pick_wpr(int64_t rows, int64_t D) {
  int wpr = 1;
  while (wpr < 8 && D > (int64_t)wpr * 64 * 8 * 4) wpr *= 2;
  if (rows < 2048 && D >= 2048 && wpr < 2) wpr = 2;
  if (rows < 512 && D >= 2048 && wpr < 4) wpr = 4;
  if (rows < 128 && D >= 2048) wpr = 8;  // 64 x 4096: 4.5 -> 3.6 us
  return wpr;
}

int block_threads(int wpr) { return wpr <= 4 ? 256 : 64 * wpr; }
int rows_per_block(int wpr) { return wpr <= 4 ? 4 / wpr : 1; }

#define FRT_NV_SWITCH(NVV, ...)                    \
  switch (NVV) {                                   \
    case 1: { constexpr int NV = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int NV = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int NV = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int NV = 4; __VA_ARGS__; } break; \
    case 5: { constexpr int NV = 5; __VA_ARGS__; } break; \
    case 6: { constexpr int NV = 6; __VA_ARGS__; } break; \
    case 7: { constexpr int NV = 7; __VA_ARGS__; } break; \
    case 8: { constexpr int NV = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;          \
  }

#define FRT_NV2_SWITCH(NVV, ...)                   \
  switch (NVV) {                                   \
    case 2: { constexpr int NV = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int NV = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int NV = 8; __VA_ARGS__; } break; \
    case 16: { constexpr int NV = 16; __VA_ARGS__; } break; \
    case 32: { constexpr int NV = 32; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;          \
  }

int pow2_slots(int64_t n) {
  int p = 2;
  while (p < n) p <<= 1;
  return p;
}

#define FRT_WPR_SWITCH(W, ...)                     \
  switch (W) {                                     \
    case 1: { constexpr int WPR = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int WPR = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int WPR = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int WPR = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;          \
  }

}  // namespace

hipError_t launch_ada_norm(const AdaArgs& a, bool vec8, hipStream_t st) {
  const int vec = vec8 ? 8 : 2;
  const int wpr = pick_wpr(a.M, a.D);
  const int64_t nvec = a.D / vec;
  const int nv = (int)((nvec + 64 * wpr - 1) / (64 * wpr));
  const int rpb = rows_per_block(wpr);
  const dim3 grid((unsigned)((a.M + rpb - 1) / rpb));
  const dim3 block((unsigned)block_threads(wpr));
  if (vec8) {
    FRT_WPR_SWITCH(wpr, FRT_NV_SWITCH(nv, hipLaunchKernelGGL((ada_norm_kernel<WPR, NV, 8>), grid, block, 0, st, a)))
  } else {
    // 4-byte path (unaligned or D % 8 != 0): one row per block, 4 waves,
    // up to 32 two-element slots per lane
    const int nv2 = pow2_slots((nvec + 255) / 256);
    const dim3 grid4((unsigned)a.M);
    FRT_NV2_SWITCH(nv2, hipLaunchKernelGGL((ada_norm_kernel<4, NV, 2>), grid4, dim3(256), 0, st, a))
  }
  return hipGetLastError();
}

hipError_t launch_ada_norm_mxfp4(const AdaArgs& a, hipStream_t st) {
  const int wpr = pick_wpr(a.M, a.D);
  const int64_t nvec = a.D / 8;
  const int nv = (int)((nvec + 64 * wpr - 1) / (64 * wpr));
  const int rpb = rows_per_block(wpr);
  const dim3 grid((unsigned)((a.M + rpb - 1) / rpb));
  const dim3 block((unsigned)block_threads(wpr));
  FRT_WPR_SWITCH(wpr, FRT_NV_SWITCH(nv, hipLaunchKernelGGL((ada_norm_kernel<WPR, NV, 8, true>), grid, block, 0, st, a)))
  return hipGetLastError();
}

hipError_t launch_ptok_norm(const PtokArgs& a, bool vec8, hipStream_t st) {
  const int wpr = pick_wpr(a.R, a.D);
  if (vec8) {
    const int64_t nvec = a.D / 8;
    const int nv = (int)((nvec + 64 * wpr - 1) / (64 * wpr));
    const int rpb = rows_per_block(wpr);
    const dim3 grid((unsigned)((a.R + rpb - 1) / rpb));
    const dim3 block((unsigned)block_threads(wpr));
    FRT_WPR_SWITCH(wpr, FRT_NV_SWITCH(nv, hipLaunchKernelGGL((ptok_norm_kernel<WPR, NV, 8>), grid, block, 0, st, a)))
  } else {
    const int64_t nvec = a.D / 2;
    const int nv2 = pow2_slots((nvec + 255) / 256);
    const dim3 grid4((unsigned)a.R);
    FRT_NV2_SWITCH(nv2, hipLaunchKernelGGL((ptok_norm_kernel<4, NV, 2>), grid4, dim3(256), 0, st, a))
  }
  return hipGetLastError();
}

}  // namespace frt
