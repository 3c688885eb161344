// Packed FP8 GEMM with dequant + bias + column-split epilogue on gfx950.
//
// out[m, n] = bf16(fl32(alpha * sum_k x8[m,k] * W8[n,k]) + bias[n]) written
// into the split s that owns column n (flashrt-structures 0.2.0,
// impls/qkv_pack/fp8_static.py `PackedLinear._run`; alpha = act_scale *
// w_scale as folded in impls/adarms_stack/fp8_chain.py `_quantize`).
//
// Both operands are K-contiguous ("TN"). The main loop runs on the CDNA4
// FP8 matrix cores, v_mfma_f32_32x32x64_f8f6f4 (A = 32 rows of x8, B = 32
// rows of W8, 64-deep K step, fp32 accumulate).
//
// Tiles are staged through LDS with direct buffer->LDS loads
// (buffer_load_dwordx4 ... lds): each load instruction of a wave writes one
// 1 KiB "half-fragment" = for the 64 lanes of the consuming MFMA, lane l's
// 16 bytes (row l % 32, K bytes [h*32 + (l/32)*16, +16) of the 64-deep step).
// The consumer reads it back with one ds_read_b128 per lane at
// base + l*16: consecutive lanes, consecutive addresses, no bank conflicts.
// Each lane's two halves form its 32-byte MFMA operand. A and B use the same
// per-lane K assignment, so whatever K order the matrix core applies inside
// the instruction, the products pair up correctly.
//
// Rows beyond M (or N) and K chunks beyond K read zeros: their buffer offset
// is pushed past the buffer's record count, which the hardware turns into a
// zero fill.
//
// Block order is XCD-aware: the dispatcher places block b on XCD b % 8, so
// the logical tile index gives each XCD a contiguous run of tiles, and runs
// are rastered in groups of GM tile-rows so that the tiles resident on one
// XCD share A and B panels in that XCD's L2.
#include "frt_device.h"
#include "frt_internal.h"

namespace frt {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOOB = 0x80000000u;  // offset past any record count

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // flags: default data format for raw buffer loads on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// vmcnt wait immediate for gfx9 (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

struct TileXY {
  int tm, tn;
};

// XCD-aware, L2-grouped tile order (see the file comment).
__device__ __forceinline__ TileXY tile_of(int b, int tiles_m, int tiles_n, int gm) {
  const int T = tiles_m * tiles_n;
  const int xcd = b & 7, q = b >> 3;
  const int per = T >> 3, rem = T & 7;
  const int L = xcd * per + min(xcd, rem) + q;
  const int gsz = gm * tiles_n;
  const int g = L / gsz;
  const int first = g * gm;
  const int rows = min(gm, tiles_m - first);
  const int within = L - g * gsz;
  return TileXY{first + within % rows, within / rows};
}

}  // namespace

// BM x BN block tile, WM x WN per wave, 64-deep K steps, NSTAGE-deep LDS
// ring.
template <int BM, int BN, int WM, int WN, int NSTAGE, int GM>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_tiled_kernel(GemmArgs a) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NW = (BM / WM) * WAVES_N;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int A_HF = (BM / 32) * 2;  // 1 KiB half-fragments per stage
  constexpr int B_HF = (BN / 32) * 2;
  constexpr int HF = A_HF + B_HF;
  static_assert(HF % NW == 0, "loads must split evenly over the waves");
  constexpr int LPW = HF / NW;  // load instructions per wave per stage
  constexpr int STAGE = HF * 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * STAGE];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const TileXY t = tile_of(blockIdx.x, tiles_m, tiles_n, GM);
  const int m0 = t.tm * BM, n0 = t.tn * BN;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

  const uint32_t x_bytes = (uint32_t)((int64_t)(a.M - 1) * a.ld_x + a.K);
  const uint32_t w_bytes = (uint32_t)((int64_t)a.N * a.K);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, w_bytes);

  // per-lane source offsets of this wave's LPW half-fragments, K step 0
  uint32_t off[LPW];
  bool isA[LPW];
  int kin[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int f = wave + j * NW;
    const bool A = f < A_HF;
    const int g = A ? f : f - A_HF;
    const int sub = g >> 1, h = g & 1;
    const int r = (A ? m0 : n0) + sub * 32 + (lane & 31);
    const int kb = h * 32 + (lane >> 5) * 16;
    const bool ok = r < (A ? a.M : a.N);
    isA[j] = A;
    kin[j] = kb;
    off[j] = ok ? (uint32_t)(A ? (int64_t)r * a.ld_x : (int64_t)r * a.K) + kb : kOOB;
  }

  auto issue = [&](int kt, int stage) {
    const int k0 = kt * 64;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int f = wave + j * NW;
      uint8_t* dst = smem + stage * STAGE + f * 1024;
      const uint32_t o = (off[j] == kOOB || k0 + kin[j] >= a.K) ? kOOB : off[j] + k0;
      if (isA[j])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
    }
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = (a.K + 63) / 64;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KT) issue(s, s);

  for (int kt = 0; kt < KT; ++kt) {
    const int pre = kt + NSTAGE - 1;
    if (pre < KT) issue(pre, pre % NSTAGE);
    // wait until this K step's loads have landed (later steps may fly)
    const int ahead = min(KT - 1 - kt, NSTAGE - 1);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPW));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    const uint8_t* sb = smem + (kt % NSTAGE) * STAGE;
    v8i af[MI], bf[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int sub = (wm0 >> 5) + i;
      const v4i lo = *reinterpret_cast<const v4i*>(sb + (2 * sub) * 1024 + lane * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(sb + (2 * sub + 1) * 1024 + lane * 16);
      af[i] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int sub = (wn0 >> 5) + j;
      const v4i lo = *reinterpret_cast<const v4i*>(sb + (A_HF + 2 * sub) * 1024 + lane * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(sb + (A_HF + 2 * sub + 1) * 1024 + lane * 16);
      bf[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, 0,
                                                                    0, 0);
    __syncthreads();  // every wave is done with this stage before refill
  }

  // ---- epilogue: alpha * acc + bias, column split, bf16 (or fp32) ----
  const float alpha = (*a.act_scale) * (*a.w_scale);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn0 + j * 32 + (lane & 31);
    if (n >= a.N) continue;
    // the split that owns column n (uniform loop, per-lane selects)
    uint8_t* base = reinterpret_cast<uint8_t*>(a.sp.ptr[0]);
    int64_t ld = a.sp.ld[0];
    int off0 = 0;
#pragma unroll
    for (int s = 1; s < FRT_MAX_SPLITS; ++s) {
      if (s < a.sp.n && n >= a.sp.off[s]) {
        base = reinterpret_cast<uint8_t*>(a.sp.ptr[s]);
        ld = a.sp.ld[s];
        off0 = a.sp.off[s];
      }
    }
    const float b = a.bias != nullptr ? bf16f(a.bias[n]) : 0.0f;
    const int col = n - off0;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < a.M) {
          const float v = alpha * acc[i][j][r] + b;
          if (a.out_f32)
            reinterpret_cast<float*>(base)[(int64_t)m * ld + col] = v;
          else
            reinterpret_cast<uint16_t*>(base)[(int64_t)m * ld + col] = (uint16_t)f2bf(v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)M; (void)N; (void)K;
  return 0;
}

namespace {

template <int BM, int BN, int WM, int WN, int NSTAGE, int GM>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WM, WN, NSTAGE, GM>), dim3(tiles), dim3(threads), 0, st,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M >= 512) return launch_tiled<256, 256, 128, 128, 2, 4>(a, st);
  if (a.M > 64) return launch_tiled<128, 128, 64, 64, 2, 2>(a, st);
  if (a.M > 32) return launch_tiled<64, 64, 32, 32, 2, 1>(a, st);
  return launch_tiled<32, 64, 32, 32, 2, 1>(a, st);
}

}  // namespace frt
