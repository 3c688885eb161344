// QKV split + adjacent-pair RoPE + KV-cache write, and the pack-time pair
// interleave of the q/k projection rows.
//
// flashrt-structures 0.2.0, impls/adarms_stack/fp8_chain.py: the module
// docstring (the host rotates pairs (i, i + hd/2); the split kernel rotates
// adjacent pairs, with the q/k rows permuted at pack time so that position
// 2i holds dimension i and 2i + 1 holds i + hd/2), `_build_rope` (bf16
// table [S, hd], cosine at even and sine at odd positions) and `_make_run`
// (the split call on the merged [1, S, (nh + 2kv) hd] QKV output, q out, the
// suffix K/V written behind P prefix rows of [1, T, kv, hd] caches).
//
// For an adjacent pair (a, b) and the table pair (c, s) of its token:
//   a' = a c - b s,  b' = b c + a s,  rounded once to bf16.
// Both products of two bf16 values are exact in fp32, so a' and b' are the
// single fp32 rounding of the exact result however the two terms are
// combined.
#include "frt_device.h"
#include "frt_internal.h"

namespace frt {

namespace {

// One thread per 8 columns (4 pairs) of one token row.
template <int VEC>
__global__ __launch_bounds__(256) void rope_split_kernel(RopeArgs a) {
  const int ncol = (a.nh + 2 * a.kv) * a.hd;
  const int nq = a.nh * a.hd, nk = a.kv * a.hd;
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * VEC;
  if (c0 >= ncol) return;
  for (int64_t m = blockIdx.y; m < a.S; m += gridDim.y) {
    const uint16_t* src = a.qkv + m * a.ld_qkv + c0;
    uint16_t* dst;
    bool rot = true;
    if (c0 < nq) {
      dst = a.q_out + m * nq + c0;
    } else if (c0 < nq + nk) {
      dst = a.k_cache + (a.P + m) * nk + (c0 - nq);
    } else {
      dst = a.v_cache + (a.P + m) * nk + (c0 - nq - nk);
      rot = false;
    }
    const int d0 = c0 % a.hd;  // even: VEC-aligned columns within a head
    const uint16_t* rp = a.rope + m * a.hd + d0;
    uint32_t w[VEC / 2], r[VEC / 2];
    if constexpr (VEC == 8) {
      const uint4 t = *reinterpret_cast<const uint4*>(src);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(src);
    }
    if (rot) {
      if constexpr (VEC == 8) {
        const uint4 t = *reinterpret_cast<const uint4*>(rp);
        r[0] = t.x; r[1] = t.y; r[2] = t.z; r[3] = t.w;
      } else {
        r[0] = *reinterpret_cast<const uint32_t*>(rp);
      }
#pragma unroll
      for (int p = 0; p < VEC / 2; ++p) {
        const float x0 = bf16lo(w[p]), x1 = bf16hi(w[p]);
        const float c = bf16lo(r[p]), s = bf16hi(r[p]);
        w[p] = pack_bf2(__builtin_fmaf(x0, c, -(x1 * s)), __builtin_fmaf(x1, c, x0 * s));
      }
    }
    if constexpr (VEC == 8)
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    else
      *reinterpret_cast<uint32_t*>(dst) = w[0];
  }
}

// dst row h*hd + j = src row h*hd + perm(j), perm(2i) = i,
// perm(2i + 1) = i + hd/2; one thread per 8 (or 1) elements of a row.
template <int VEC>
__global__ __launch_bounds__(256) void interleave_kernel(const uint16_t* src, uint16_t* dst, int nheads, int hd,
                                                         int64_t K) {
  const int64_t nv = K / VEC;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= nv) return;
  const int half = hd / 2;
  for (int64_t row = blockIdx.y; row < (int64_t)nheads * hd; row += gridDim.y) {
    const int64_t h = row / hd;
    const int j = (int)(row - h * hd);
    const int64_t srow = h * hd + ((j & 1) ? half + (j >> 1) : (j >> 1));
    if constexpr (VEC == 8)
      reinterpret_cast<uint4*>(dst + row * K)[v] = reinterpret_cast<const uint4*>(src + srow * K)[v];
    else
      dst[row * K + v] = src[srow * K + v];
  }
}

}  // namespace

hipError_t launch_rope_split(const RopeArgs& a, int vec, hipStream_t st) {
  const int ncol = (a.nh + 2 * a.kv) * a.hd;
  const int threads_per_row = (ncol + vec - 1) / vec;
  const dim3 grid((unsigned)((threads_per_row + 255) / 256), (unsigned)(a.S < 65535 ? a.S : 65535));
  if (vec == 8)
    hipLaunchKernelGGL((rope_split_kernel<8>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((rope_split_kernel<2>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_interleave(const uint16_t* src, uint16_t* dst, int nheads, int hd, int64_t K, int vec,
                             hipStream_t st) {
  const int64_t nv = K / vec;
  const int64_t rows = (int64_t)nheads * hd;
  const dim3 grid((unsigned)((nv + 255) / 256), (unsigned)(rows < 65535 ? rows : 65535));
  if (vec == 8)
    hipLaunchKernelGGL((interleave_kernel<8>), grid, dim3(256), 0, st, src, dst, nheads, hd, K);
  else
    hipLaunchKernelGGL((interleave_kernel<1>), grid, dim3(256), 0, st, src, dst, nheads, hd, K);
  return hipGetLastError();
}

}  // namespace frt
