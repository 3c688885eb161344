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
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "frt_device.h"
#include "frt_internal.h"

namespace frt {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOOB = 0x80000000u;  // offset past any record count
// cache-policy operand of buffer loads/stores: sc1, i.e. coherent at agent
// scope (the instruction form of a relaxed agent-scope atomic access: stores
// are written through to the device-coherent level, loads never hit a line
// another XCD's writes could have left stale)
constexpr int kCoherent = 0x10;

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

// vmcnt(n) together with lgkmcnt(0) (expcnt left at its maximum)
__device__ __forceinline__ constexpr int vm_lgkm0_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4);
}

// BM x BN block tile, WM x WN per wave, 64-deep K steps, NSTAGE-deep LDS
// ring (NSTAGE - 1 K steps in flight).
//
// Per K step kt a wave: issues the global->LDS loads of step kt+NSTAGE-1
// (into the slot step kt-1 used), runs the first MFMAs of step kt on
// fragments already in registers, waits until step kt+1's loads have
// landed (its own: vmcnt; everyone's: one s_barrier), then reads step
// kt+1's fragments into the other register set while the remaining MFMAs
// of step kt run. One barrier per K step; the slot being refilled was last
// read two barriers earlier.
//
// PP = false (no fragment ping-pong): the wave waits for step kt itself,
// passes the barrier, refills the slot step kt-1 used, then reads step kt's
// fragments and runs its MFMAs; half the fragment registers.
template <int BM, int BN, int WM, int WN, int NSTAGE, int GM, bool PP, bool KTAIL>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_tiled_kernel(GemmArgs a) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NW = (BM / WM) * WAVES_N;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int A_HF = (BM / 32) * 2;  // 1 KiB half-fragments per stage
  constexpr int B_HF = (BN / 32) * 2;
  constexpr int HF = A_HF + B_HF;
  static_assert(HF % NW == 0, "loads must split evenly over the waves");
  static_assert(NSTAGE >= 2, "at least double buffering");
  constexpr int LPW = HF / NW;  // load instructions per wave per stage
  constexpr int STAGE = HF * 1024;
  constexpr int PRE = MI * NJ >= 8 ? 4 : (MI * NJ >= 4 ? 2 : 1);  // MFMAs before the barrier
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
  // (K byte within the step: h * 32 + (lane / 32) * 16, h = f & 1)
  uint32_t off[LPW];
  const int kl = (lane >> 5) * 16;
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int f = wave + j * NW;
    const bool A = f < A_HF;
    const int g = A ? f : f - A_HF;
    const int sub = g >> 1, h = g & 1;
    const int r = (A ? m0 : n0) + sub * 32 + (lane & 31);
    const bool ok = r < (A ? a.M : a.N);
    off[j] = ok ? (uint32_t)(A ? (int64_t)r * a.ld_x : (int64_t)r * a.K) + h * 32 + kl : kOOB;
  }

  const int KT = (a.K + 63) / 64;
  auto issue = [&](int kt) {
    const int k0 = kt * 64;
    uint8_t* sbase = smem + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int f = wave + j * NW;  // f < A_HF is uniform per (wave, j)
      uint8_t* dst = sbase + f * 1024;
      uint32_t o = off[j] + k0;  // kOOB + k0 stays past every record count
      if constexpr (KTAIL) {
        if (k0 + (f & 1) * 32 + kl >= a.K) o = kOOB;
      }
      if (f < A_HF)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
    }
  };
  auto read_frags = [&](int kt, v8i* af, v8i* bf) {
    const uint8_t* sb = smem + (kt % NSTAGE) * STAGE;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int sub = (wn0 >> 5) + j;
      const v4i lo = *reinterpret_cast<const v4i*>(sb + (A_HF + 2 * sub) * 1024 + lane * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(sb + (A_HF + 2 * sub + 1) * 1024 + lane * 16);
      bf[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int sub = (wm0 >> 5) + i;
      const v4i lo = *reinterpret_cast<const v4i*>(sb + (2 * sub) * 1024 + lane * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(sb + (2 * sub + 1) * 1024 + lane * 16);
      af[i] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // wait (own loads) until at most `ahead` later stages are in flight, and
  // for every LDS read; then the block barrier
  auto sync_stage = [&](int ahead) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NSTAGE >= 4) {
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(2 * LPW));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(LPW));
      else __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
    } else if constexpr (NSTAGE == 3) {
      if (ahead >= 1) __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(LPW));
      else __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
    } else {
      __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // prologue: NSTAGE-1 steps in flight
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < KT) issue(s);

  if constexpr (!PP) {
    v8i fa[MI], fb[NJ];
    for (int kt = 0; kt < KT; ++kt) {
      // step kt landed (later steps may fly); everyone is past step kt-1
      sync_stage(min(KT - 1 - kt, NSTAGE - 2));
      if (kt + NSTAGE - 1 < KT) issue(kt + NSTAGE - 1);
      read_frags(kt, fa, fb);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  } else {
  // step 0 landed and read
  sync_stage(min(KT - 1, NSTAGE - 2));
  v8i fa0[MI], fb0[NJ], fa1[MI], fb1[NJ];
  read_frags(0, fa0, fb0);

  auto kstep = [&](int kt, v8i* ca, v8i* cb, v8i* na, v8i* nb) {
    if (kt + NSTAGE - 1 < KT) issue(kt + NSTAGE - 1);
    // first MFMAs of step kt (their fragments are already in registers)
#pragma unroll
    for (int q = 0; q < PRE; ++q) {
      const int i = q / NJ, j = q % NJ;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ca[i], cb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
    if (kt + 1 < KT) {
      // stages still allowed in flight beyond kt+1
      sync_stage(min(KT - 2 - kt, NSTAGE - 2));
      read_frags(kt + 1, na, nb);
    }
#pragma unroll
    for (int q = PRE; q < MI * NJ; ++q) {
      const int i = q / NJ, j = q % NJ;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ca[i], cb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  };

  for (int kt = 0; kt < KT; kt += 2) {
    kstep(kt, fa0, fb0, fa1, fb1);
    if (kt + 1 < KT) kstep(kt + 1, fa1, fb1, fa0, fb0);
  }
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

// ---------------------------------------------------------------------------
// Large-tile kernel: 128-deep K stages staged as full 128-byte row segments.
//
// LDS holds each stage row-major, one 128-byte row segment per tile row, with
// the eight 16-byte chunks of row r stored at chunk position
// c ^ ((r >> 1) & 7) (an XOR swizzle). A direct buffer->LDS load
// instruction of a wave therefore covers 8 rows x 128 contiguous bytes (whole
// cache lines, 8 requests per KiB instead of 32), and each lane's destination
// stays lane-contiguous as the instruction requires: lane L writes chunk
// position L % 8 of row L / 8, so it fetches global chunk
// (L % 8) ^ ((row >> 1) & 7). A 32x32x64 operand read (row l % 32, K bytes
// [s*64 + (l/32)*32, +32)) takes chunks c0 = s*4 + (l/32)*2 and c0 + 1,
// i.e. positions c0 ^ ((l >> 1) & 7) and that ^ 1. The LDS serves a
// ds_read_b128 sixteen lanes (256 bytes, all 64 banks) at a time: sixteen
// consecutive rows fall in two 128-byte halves by row parity and on eight
// distinct positions within each half, so the reads are conflict free.
//
// Two stages (BK = 128 each), one barrier per stage, after which the freed
// stage is refilled. Eight waves (two per SIMD): while one wave waits for
// its fragment reads the other wave's MFMAs keep the matrix core busy, so
// a wave holds a single fragment set (no spills at 2 waves per SIMD).
template <int BM, int BN, int WM, int WN, int NS, int GM, bool KTAIL, int NSUB = 1, bool SK = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_big_kernel(GemmArgs a) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NW = (BM / WM) * WAVES_N;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int LOADS = ROWS / 8;  // 1 KiB load instructions per stage
  static_assert(LOADS % NW == 0, "loads must split evenly over the waves");
  constexpr int LPW = LOADS / NW;
  constexpr int SUBB = ROWS * 128;     // one 128-deep sub-buffer
  constexpr int STAGE = NSUB * SUBB;   // one stage = NSUB sub-buffers
  constexpr int KST = 128 * NSUB;      // K bytes per stage
  static_assert(NS >= 2 && NSUB * LPW * (NS - 2) <= 63, "ring depth vs vmcnt range");
  static_assert(NS * STAGE <= 160 * 1024, "ring exceeds LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  // split-K decomposition: blocks [0, n_full) own whole tiles; each of the
  // remaining tiles is split along K over nsplit consecutive blocks
  int tile_id = blockIdx.x, zsplit = 0, S_eff = 1, tail = 0;
  if constexpr (SK) {
    if ((int)blockIdx.x >= a.n_full) {
      const int q = blockIdx.x - a.n_full;
      tail = q / a.nsplit;
      zsplit = q % a.nsplit;
      S_eff = a.nsplit;
      tile_id = a.n_full + tail;
    }
  }
  const TileXY t = tile_of(tile_id, tiles_m, tiles_n, GM);
  const int m0 = t.tm * BM, n0 = t.tn * BN;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

  const uint32_t x_bytes = (uint32_t)((int64_t)(a.M - 1) * a.ld_x + a.K);
  const uint32_t w_bytes = (uint32_t)((int64_t)a.N * a.K);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, w_bytes);

  // this wave's load instructions: tile rows [8u, 8u + 8), u = wave + j*NW.
  // One base offset per operand; instruction j adds a uniform multiple of
  // the row stride. A row past M (N) lands past the buffer's record count
  // ((M-1)*ld_x + K, resp. N*K, with ld_x >= K), which the hardware turns
  // into a zero fill, so no per-load bound registers are kept.
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "A and B loads split evenly");
  constexpr int LPA = BM / (8 * NW);  // the first LPA loads of a wave are A rows
  const int lrow = lane >> 3;
  // global chunk this lane fetches: rows 8u + lrow with u = wave + j*NW and
  // NW even, so (row >> 1) & 7 = ((wave & 1) << 2) | (lrow >> 1) for every j
  static_assert(NW % 2 == 0, "row swizzle assumes an even wave count");
  const int cch = (lane & 7) ^ (((wave & 1) << 2) | (lrow >> 1));
  // split-K: this block covers K bytes [kb, kb + kc) (kc a multiple of
  // KST; the planner leaves no split empty)
  const int kb = S_eff > 1 ? zsplit * a.kc : 0;
  const int klen = S_eff > 1 ? min(a.kc, a.K - kb) : a.K;
  const uint32_t offA = (uint32_t)((int64_t)(m0 + wave * 8 + lrow) * a.ld_x) + kb + cch * 16;
  const uint32_t offB = (uint32_t)((int64_t)(n0 + wave * 8 + lrow) * a.K) + kb + cch * 16;
  const uint32_t stepA = (uint32_t)(8 * NW) * (uint32_t)a.ld_x;
  const uint32_t stepB = (uint32_t)(8 * NW) * (uint32_t)a.K;
  const int KT = (klen + KST - 1) / KST;
  // slot SL (= step mod NS) is a compile-time constant in every use, so all
  // LDS addresses are one lane base plus immediates
  auto issue = [&](int kt, auto SLC) {
    constexpr int SL = decltype(SLC)::value;
#pragma unroll
    for (int q = 0; q < NSUB; ++q) {
      const int k0 = kt * KST + q * 128;
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int u = wave + j * NW;
        uint8_t* dst = smem + SL * STAGE + q * SUBB + u * 1024;
        const bool A = j < LPA;
        uint32_t o = A ? offA + j * stepA + k0 : offB + (j - LPA) * stepB + k0;
        if constexpr (KTAIL) {
          if (k0 + cch * 16 >= klen) o = kOOB;
        }
        if (A)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
      }
    }
  };
  // operand read of substep SUB from slot SL: two 16-byte chunks per lane
  const int lrow32 = lane & 31;
  const int sw = (lrow32 >> 1) & 7;  // (row >> 1) & 7 for rows 32k + lrow32
  const uint8_t* lbase0 = smem + lrow32 * 128 + ((((lane >> 5) * 2) ^ sw) * 16);
  const uint8_t* lbase1 = smem + lrow32 * 128 + ((((lane >> 5) * 2 + 4) ^ sw) * 16);
  auto read_frags = [&](auto SLC, auto SUBC, v8i* af, v8i* bf) {
    constexpr int SL = decltype(SLC)::value, SUB = decltype(SUBC)::value;
    const uint8_t* lb = ((SUB & 1) ? lbase1 : lbase0) + SL * STAGE + (SUB >> 1) * SUBB;
    // the second chunk sits at position ^ 1, i.e. +16 or -16 bytes
    const int d1 = (sw & 1) ? -16 : 16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint8_t* rowp = lb + (BM + wn0 + j * 32) * 128;
      const v4i lo = *reinterpret_cast<const v4i*>(rowp);
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + d1);
      bf[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint8_t* rowp = lb + (wm0 + i * 32) * 128;
      const v4i lo = *reinterpret_cast<const v4i*>(rowp);
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + d1);
      af[i] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // own loads: at most `ahead` later stages still in flight; every LDS read
  // done; then the block barrier (s_waitcnt takes an immediate: one case per
  // possible depth)
  auto sync_stage = [&](int ahead) {
    __builtin_amdgcn_sched_barrier(0);
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((ahead == I ? (__builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(NSUB * LPW * I)), 0) : 0), ...);
    }(std::make_integer_sequence<int, NS - 1>{});
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  using I0 = std::integral_constant<int, 0>;
  // Small wave tiles read every 64-deep substep of a stage right after the
  // barrier (one LDS round trip per stage) and alternate between two
  // independent accumulator sets, so consecutive MFMAs do not wait on each
  // other; large wave tiles reuse one fragment set and one accumulator set.
  constexpr int KSUB = 2 * NSUB;
  constexpr bool ALL = MI * NJ * KSUB <= 8;
  constexpr int NACC = (ALL && KSUB >= 2) ? 2 : 1;
  constexpr int NF = ALL ? KSUB : 1;
  v8i fa[NF][MI], fb[NF][NJ];
  v16f acc2[NACC > 1 ? MI : 1][NACC > 1 ? NJ : 1];
  if constexpr (NACC > 1) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc2[i][j][r] = 0.0f;
  }
  auto mfmas = [&](const v8i* af, const v8i* bf, auto ACC) {
#pragma unroll
    for (int q = 0; q < MI * NJ; ++q) {
      const int i = q / NJ, j = q % NJ;
      if constexpr (decltype(ACC)::value == 0)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
      else
        acc2[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc2[i][j], 0, 0, 0, 0, 0, 0);
    }
  };
  auto read_all = [&](auto SLC) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (read_frags(SLC, std::integral_constant<int, U>{}, fa[U], fb[U]), ...);
    }(std::make_integer_sequence<int, NF>{});
  };
  // one stage kt held in slot SL = kt % NS. The slot refilled first,
  // (kt - 1) % NS, was last read before the previous barrier.
  auto stage = [&](int kt, auto SLC) {
    constexpr int SL = decltype(SLC)::value;
    using PV = std::integral_constant<int, (SL + NS - 1) % NS>;
    using NX = std::integral_constant<int, (SL + 1) % NS>;
    if (kt + NS - 1 < KT) issue(kt + NS - 1, PV{});
    if constexpr (ALL) {
      [&]<int... U>(std::integer_sequence<int, U...>) {
        (mfmas(fa[U], fb[U], std::integral_constant<int, U % NACC>{}), ...);
      }(std::make_integer_sequence<int, KSUB>{});
    } else {
      [&]<int... U>(std::integer_sequence<int, U...>) {
        ((U > 0 ? (read_frags(SLC, std::integral_constant<int, U>{}, fa[0], fb[0]), 0) : 0,
          mfmas(fa[0], fb[0], std::integral_constant<int, 0>{})), ...);
      }(std::make_integer_sequence<int, KSUB>{});
    }
    if (kt + 1 < KT) {
      // step kt+1 landed everywhere (later ones may fly); step kt fully read
      sync_stage(min(KT - 2 - kt, NS - 2));
      if constexpr (ALL) read_all(NX{});
      else read_frags(NX{}, I0{}, fa[0], fb[0]);
    }
  };
  auto ring = [&](int kt0, auto... SLs) {
    int kt = kt0;
    ((kt < KT ? (stage(kt, SLs), ++kt) : 0), ...);
  };

  // prologue: steps 0 .. NS-2 in flight (slot index = step)
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((I < KT ? (issue(I, std::integral_constant<int, I>{}), 0) : 0), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
  sync_stage(min(KT - 1, NS - 2));
  if constexpr (ALL) read_all(I0{});
  else read_frags(I0{}, I0{}, fa[0], fb[0]);
  for (int kt = 0; kt < KT; kt += NS) {
    [&]<int... S>(std::integer_sequence<int, S...>) {
      ring(kt, std::integral_constant<int, S>{}...);
    }(std::make_integer_sequence<int, NS>{});
  }
  if constexpr (NACC > 1) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] += acc2[i][j];
  }

  if (SK && S_eff > 1) {
    // Split-K: every split stores its fp32 partial tile in fragment order
    // (lane-contiguous 16-byte groups, so each store instruction writes one
    // contiguous KiB) with agent-coherent stores, then bumps the tile's
    // arrival counter; the last block to arrive sums the partials of
    // splits 0..S-1 in that order (the result does not depend on which
    // block finishes last), resets the counter and runs the epilogue.
    __shared__ int last_flag;
    constexpr int FR = MI * NJ * 4;        // 16-byte groups per lane
    constexpr int TILE_B = BM * BN * 4;    // bytes per partial tile
    const int S = S_eff;
    const int n_tail = tiles_m * tiles_n - a.n_full;
    const uint32_t wave_off = (uint32_t)wave * (FR * 1024) + lane * 16;
    const uint32_t plane = (uint32_t)n_tail * TILE_B;
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.ws, plane * (uint32_t)S);
    const uint32_t tile_off = (uint32_t)tail * TILE_B + wave_off;
    {
      const uint32_t o = (uint32_t)zsplit * plane + tile_off;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f v = (v4f){acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), pr,
                                                   o + ((i * NJ + j) * 4 + g) * 1024, 0, kCoherent);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);  // partial stores performed at agent scope
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* c = a.cnt + tail;
      const unsigned prev = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = prev == (unsigned)(S - 1);
      if (last_flag) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // one accumulator row-block (NJ tiles) at a time, splits in order
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      for (int z = 0; z < S; ++z) {
        const uint32_t o = (uint32_t)z * plane + tile_off;
        v4i part[NJ][4];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            part[j][g] = __builtin_amdgcn_raw_buffer_load_b128(pr, o + ((i * NJ + j) * 4 + g) * 1024, 0, kCoherent);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f v = __builtin_bit_cast(v4f, part[j][g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] += v[e];
          }
      }
    }
  }

  // ---- epilogue: alpha * acc + bias, column split, bf16 (or fp32) ----
  const float alpha = (*a.act_scale) * (*a.w_scale);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = n0 + wn0 + j * 32 + (lane & 31);
    if (n >= a.N) continue;
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

// ---------------------------------------------------------------------------
// Skinny kernel (M <= 64): weight streaming with split-K.
//
// A block owns 64 rows of W8 (16 per wave) and one K range of KS = 128*NCH
// bytes (split s = blockIdx.y of S). Each wave loads its 16 W rows for the
// whole K range straight into registers up front (NCH*2 loads of 16 bytes
// per lane, all in flight at once); there is no barrier in the K loop. The
// x rows (MG*16 rows, zero beyond M) of the K range are staged once in LDS
// and read as MFMA operands; v_mfma_f32_16x16x128_f8f6f4 with A = 16 x rows,
// B = 16 W rows, fp32 accumulate.
//
// Operand K order: within a 128-byte chunk, lane l (row l % 16, group
// g = l / 16) holds bytes [g*16, +16) and [64 + g*16, +16), for W and x
// alike; a W load instruction therefore reads 64 contiguous bytes of each
// of 16 rows. x rows in LDS are KS bytes long with 16-byte chunk q of row r
// stored at position q ^ (r & 15): the 16 rows a ds_read_b128 touches sit
// on 16 distinct bank groups.
//
// With S > 1 every block writes its fp32 partial tile with device-coherent
// (sc1) stores, waits for them, and bumps the tile's arrival counter (device
// scope); the block that arrives last sums the S partials in split order
// (the result does not depend on arrival order), applies the epilogue and
// resets the counter to zero for the next call.
template <int MG, int NCH, bool KTAIL>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs a, int S) {
  constexpr int KS = 128 * NCH;
  constexpr int XR = MG * 16;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[XR * KS];
  __shared__ int last_flag;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int n0 = tile * 64 + wave * 16;
  const int kb = split * KS;

  // W: this wave's 16 rows, all chunks of the K range, into registers
  const uint32_t w_bytes = (uint32_t)((int64_t)a.N * a.K);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, w_bytes);
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t wrow = (uint32_t)(n0 + r16) * (uint32_t)a.K;  // rows >= N read zeros
  v4i wv[NCH][2];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = kb + c * 128 + h * 64 + g * 16;
      uint32_t o = wrow + k;
      if constexpr (KTAIL) {
        if (k >= a.K) o = kOOB;
      }
      wv[c][h] = __builtin_amdgcn_raw_buffer_load_b128(wr, o, 0, 0);
    }
  }

  // x: XR rows x KS bytes into LDS (direct loads; one row per KiB)
  {
    const uint32_t x_bytes = (uint32_t)((int64_t)(a.M - 1) * a.ld_x + a.K);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, x_bytes);
    constexpr int LOADS = XR * KS / 1024;
    constexpr int CPR = KS / 16;  // chunks per row
#pragma unroll
    for (int j = 0; j < (LOADS + 3) / 4; ++j) {
      const int u = wave + j * 4;  // KiB index in the tile
      if (LOADS % 4 == 0 || u < LOADS) {
        const int t = u * 64 + lane;  // LDS chunk index
        const int row = t / CPR, pos = t % CPR;
        const int q = pos ^ (row & 15);
        const int k = kb + q * 16;
        uint32_t o = row < a.M ? (uint32_t)((int64_t)row * a.ld_x) + k : kOOB;
        if constexpr (KTAIL) {
          if (k >= a.K) o = kOOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xs + u * 1024), 16, o, 0, 0, 0);
      }
    }
  }
  // the x loads were issued after the W loads: vmcnt counts in order, so
  // waiting for all of them also waits for W (needed soon anyway)
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
  __builtin_amdgcn_s_barrier();

  v4f acc[MG];
#pragma unroll
  for (int m = 0; m < MG; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const v8i b = (v8i){wv[c][0][0], wv[c][0][1], wv[c][0][2], wv[c][0][3],
                        wv[c][1][0], wv[c][1][1], wv[c][1][2], wv[c][1][3]};
#pragma unroll
    for (int m = 0; m < MG; ++m) {
      const int row = m * 16 + r16;
      const uint8_t* rp = xs + row * KS;
      const int q0 = (c * 8 + g) ^ r16, q1 = (c * 8 + 4 + g) ^ r16;
      const v4i lo = *reinterpret_cast<const v4i*>(rp + q0 * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(rp + q1 * 16);
      const v8i av = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, acc[m], 0, 0, 0, 0, 0, 0);
    }
  }

  // C[m][n] layout of 16x16: lane holds n = n0 + (lane % 16), m = 4*(lane/16) + r
  const int n = n0 + r16;
  if (S > 1) {
    float* ws = reinterpret_cast<float*>(a.ws);
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = m * 16 + g * 4 + r;
        if (mm < a.M && n < a.N)
          __hip_atomic_store(ws + ((int64_t)split * a.M + mm) * a.N + n, acc[m][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    __builtin_amdgcn_s_waitcnt(0);  // partial stores complete (device coherent)
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* cnt = a.cnt + tile;
      const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = (prev == (unsigned)(S - 1));
      if (last_flag) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = m * 16 + g * 4 + r;
        float v = 0.0f;
        if (mm < a.M && n < a.N) {
          for (int z = 0; z < S; ++z)
            v += __hip_atomic_load(ws + ((int64_t)z * a.M + mm) * a.N + n, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        acc[m][r] = v;
      }
  }

  if (n >= a.N) return;
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
  const float alpha = (*a.act_scale) * (*a.w_scale);
  const float bias = a.bias != nullptr ? bf16f(a.bias[n]) : 0.0f;
  const int col = n - off0;
#pragma unroll
  for (int m = 0; m < MG; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = m * 16 + g * 4 + r;
      if (mm < a.M) {
        const float v = alpha * acc[m][r] + bias;
        if (a.out_f32)
          reinterpret_cast<float*>(base)[(int64_t)mm * ld + col] = v;
        else
          reinterpret_cast<uint16_t*>(base)[(int64_t)mm * ld + col] = (uint16_t)f2bf(v);
      }
    }
}

// Epilogue of a wave's MI x NJ grid of 32x32 fp32 accumulators whose top
// left output is (mw, nw): alpha * acc + bias, written to the split that
// owns each column, bf16 (or fp32).
template <int MI, int NJ>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const v16f (&acc)[MI][NJ], int mw, int nw,
                                           int lane) {
  const float alpha = (*a.act_scale) * (*a.w_scale);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = nw + j * 32 + (lane & 31);
    if (n >= a.N) continue;
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
        const int m = mw + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
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

// ---------------------------------------------------------------------------
// 64-deep-stage kernel with double-buffered operand fragments.
//
// Each stage holds a 64-byte K slice of every tile row (row-major, 64-byte
// rows), the four 16-byte chunks of row r at positions c ^ ((r >> 2) & 3).
// One direct buffer->LDS load instruction fills 16 consecutive rows (1 KiB,
// lane L -> row L / 4, position L % 4, so it fetches global chunk
// (L % 4) ^ ((L / 4 >> 2) & 3): rows 16u..16u+15 repeat the same pattern
// for every u). A 32x32x64 operand read (row l % 32, K bytes
// [(l / 32) * 32, +32) = chunks c0 = 2 (l / 32) and c0 + 1) reads positions
// c0 ^ f and c0 ^ f ^ 1, f = (row >> 2) & 3; the sixteen lanes of one
// ds_read_b128 pass (rows r..r+15, one chunk) land on sixteen distinct
// 16-byte bank groups, so reads are conflict free.
//
// Per stage: issue the loads of the stage NS-1 ahead; wait until the next
// stage has landed (later ones stay in flight) and the block has passed a
// barrier; issue the fragment reads of the next stage into the idle register
// set; then run this stage's MFMAs from the set read one stage earlier.
// After the barrier a wave therefore never waits on LDS before its MFMAs,
// and the loads of a stage have NS-1 stages of MFMA time to land.
template <int BM, int BN, int WM, int WN, int NS, int GM, bool KTAIL>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_k64_kernel(GemmArgs a) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NW = (BM / WM) * WAVES_N;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * 64;
  static_assert(ROWS % (16 * NW) == 0 && BM % 16 == 0, "loads must split evenly over the waves");
  constexpr int LPW = ROWS / (16 * NW);  // load instructions per wave per stage
  static_assert(NS >= 2 && NS % 2 == 0, "even ring depth (register set = stage parity)");
  static_assert(LPW * (NS - 2) <= 63, "ring depth vs vmcnt range");
  static_assert(NS * STAGE <= 160 * 1024, "ring exceeds LDS");
  // one LDS array per ring slot: the compiler can then tell the direct
  // loads into one slot from the fragment reads of another, and does not
  // make the reads wait for loads still in flight to other slots
  static_assert(NS <= 8, "ring depth");
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t sm2[NS > 2 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sm3[NS > 3 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sm4[NS > 4 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sm5[NS > 5 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sm6[NS > 6 ? STAGE : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t sm7[NS > 7 ? STAGE : 1];
  auto slot = [&](auto SLC) -> uint8_t* {
    constexpr int SL = decltype(SLC)::value;
    if constexpr (SL == 0) return sm0;
    else if constexpr (SL == 1) return sm1;
    else if constexpr (SL == 2) return sm2;
    else if constexpr (SL == 3) return sm3;
    else if constexpr (SL == 4) return sm4;
    else if constexpr (SL == 5) return sm5;
    else if constexpr (SL == 6) return sm6;
    else return sm7;
  };

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

  // load j of this wave fills tile rows 16u..16u+15, u = wave + j * NW;
  // rows past M (N) fall past the record count and read zeros
  // (tile rows 0..BM-1 are A rows, BM.. are B rows: wave-uniform per load)
  const int lrow = lane >> 2;
  const int cch = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t off[LPW];
  bool isA[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r0 = (wave + j * NW) * 16;
    isA[j] = r0 < BM;
    off[j] = isA[j] ? (uint32_t)((int64_t)(m0 + r0 + lrow) * a.ld_x) + cch * 16
                    : (uint32_t)((int64_t)(n0 + r0 - BM + lrow) * a.K) + cch * 16;
  }
  const int KT = (a.K + 63) / 64;
  auto issue = [&](int kt, auto SLC) {
    const int k0 = kt * 64;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      uint8_t* dst = slot(SLC) + (wave + j * NW) * 1024;
      const bool A = isA[j];
      uint32_t o = off[j] + k0;
      if constexpr (KTAIL) {
        if (k0 + cch * 16 >= a.K) o = kOOB;
      }
      if (A)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
    }
  };
  const int lrow32 = lane & 31;
  const int f = (lrow32 >> 2) & 3;
  const int lofs = lrow32 * 64 + ((((lane >> 5) * 2) ^ f) * 16);
  const int d1 = (f & 1) ? -16 : 16;  // the second chunk sits at position ^ 1
  auto read_frags = [&](auto SLC, v8i* af, v8i* bf) {
    const uint8_t* lb = slot(SLC) + lofs;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint8_t* rowp = lb + (wm0 + i * 32) * 64;
      const v4i lo = *reinterpret_cast<const v4i*>(rowp);
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + d1);
      af[i] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint8_t* rowp = lb + (BM + wn0 + j * 32) * 64;
      const v4i lo = *reinterpret_cast<const v4i*>(rowp);
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + d1);
      bf[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // own loads: at most `ahead` later stages in flight; every LDS read done;
  // then the block barrier
  auto sync_stage = [&](int ahead) {
    __builtin_amdgcn_sched_barrier(0);
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((ahead == I ? (__builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(LPW * I)), 0) : 0), ...);
    }(std::make_integer_sequence<int, NS - 1>{});
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  v16f acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  v8i fa[2][MI], fb[2][NJ];

  auto stage = [&](int kt, auto SLC) {
    constexpr int SL = decltype(SLC)::value;
    constexpr int SET = SL & 1;
    using PV = std::integral_constant<int, (SL + NS - 1) % NS>;
    using NX = std::integral_constant<int, (SL + 1) % NS>;
    if (kt + NS - 1 < KT) issue(kt + NS - 1, PV{});
    if (kt + 1 < KT) {
      sync_stage(min(KT - 2 - kt, NS - 2));
      read_frags(NX{}, fa[SET ^ 1], fb[SET ^ 1]);
    }
#pragma unroll
    for (int q = 0; q < MI * NJ; ++q) {
      const int i = q / NJ, j = q % NJ;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[SET][i], fb[SET][j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  };
  auto ring = [&](int kt0, auto... SLs) {
    int kt = kt0;
    ((kt < KT ? (stage(kt, SLs), ++kt) : 0), ...);
  };
  // steady state: every stage issues a load and keeps NS-2 later stages in
  // flight, so the wait depth is a constant and the code is branch free
  // (the compiler then knows the previous stage's fragment reads are done
  // and does not make the MFMAs wait for the reads just issued)
  auto steady = [&](int kt, auto SLC) {
    constexpr int SL = decltype(SLC)::value;
    constexpr int SET = SL & 1;
    using PV = std::integral_constant<int, (SL + NS - 1) % NS>;
    using NX = std::integral_constant<int, (SL + 1) % NS>;
    issue(kt + NS - 1, PV{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(LPW * (NS - 2)));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(NX{}, fa[SET ^ 1], fb[SET ^ 1]);
#pragma unroll
    for (int q = 0; q < MI * NJ; ++q) {
      const int i = q / NJ, j = q % NJ;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[SET][i], fb[SET][j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  };

  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((I < KT ? (issue(I, std::integral_constant<int, I>{}), 0) : 0), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
  sync_stage(min(KT - 1, NS - 2));
  read_frags(std::integral_constant<int, 0>{}, fa[0], fb[0]);
  int kt = 0;
  for (; kt + 2 * NS - 2 < KT; kt += NS) {
    [&]<int... S>(std::integer_sequence<int, S...>) {
      (steady(kt + S, std::integral_constant<int, S>{}), ...);
    }(std::make_integer_sequence<int, NS>{});
  }
  for (; kt < KT; kt += NS) {
    [&]<int... S>(std::integer_sequence<int, S...>) {
      ring(kt, std::integral_constant<int, S>{}...);
    }(std::make_integer_sequence<int, NS>{});
  }
  store_tile<MI, NJ>(a, acc, m0 + wm0, n0 + wn0, lane);
}

// ------------------------------------------------------------------ launch

// ---- split-K plan of the skinny kernel and its workspace ----------------
// Workspace = a fixed 64 KiB region of per-tile arrival counters (zero at
// rest) followed by S fp32 partial planes [S][M][N].
constexpr int64_t kCounterBytes = 64 * 1024;

struct SkinnyPlan {
  int mg, nch, splits, tiles;
};

// exploration switch (0 = the default plans)
int gemm_variant() {
  static const int v = [] {
    const char* e = getenv("FRT_GEMM_VARIANT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K) {
  SkinnyPlan p{};
  p.mg = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.tiles = (int)((N + 63) / 64);
  const int kt = (int)((K + 127) / 128);
  static const int force = [] {
    const char* e = getenv("FRT_SKINNY_NCH");
    return e ? atoi(e) : 0;
  }();
  if (force == 2 || force == 4 || force == 8) {
    p.nch = force;
  } else {
    p.nch = 8;
    // more blocks when the N tiles alone cannot fill the chip
    while (p.nch > 2 && (int64_t)p.tiles * ((kt + p.nch - 1) / p.nch) < 512) p.nch /= 2;
  }
  p.splits = (kt + p.nch - 1) / p.nch;
  return p;
}

bool use_skinny(int64_t M, int64_t N) {
  return gemm_variant() == 5 && M <= 64 && (N + 63) / 64 <= kCounterBytes / 4;
}

// ---- split-K plans of the tiled kernel ----------------------------------
// Tiles [0, n_full) run whole; each of the remaining tiles is split S ways
// along K (S consecutive blocks). Workspace = the 64 KiB counter region
// followed by S partial planes of (tiles - n_full) fp32 tiles each.
struct SkPlan {
  int bm, bn, kst;  // tile and K bytes per pipeline stage
  int S, kc, tiles, n_full;
};

// compute units of the current device (the plan fills whole rounds of them)
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// split-K configurations selectable for exploration (every tile split)
bool sk_config(int variant, SkPlan& p) {
  switch (variant) {
    case 60: p.bm = 64; p.bn = 64; p.kst = 128; return true;
    case 61: p.bm = 64; p.bn = 32; p.kst = 128; return true;
    case 62: p.bm = 64; p.bn = 128; p.kst = 128; return true;
    case 63: p.bm = 32; p.bn = 64; p.kst = 128; return true;
    case 64: p.bm = 64; p.bn = 32; p.kst = 128; return true;
    case 65: p.bm = 64; p.bn = 64; p.kst = 256; return true;
    default: return false;
  }
}

// S splits requested for the tail tiles; each split gets a whole number of
// stages and none is empty
void sk_finish(SkPlan& p, int64_t M, int64_t N, int64_t K, int S_req, int n_full) {
  const int kt = (int)((K + p.kst - 1) / p.kst);
  int S = std::max(1, std::min(S_req, kt));
  const int per = (kt + S - 1) / S;
  p.S = (kt + per - 1) / per;
  p.kc = per * p.kst;
  p.tiles = (int)(((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn));
  p.n_full = std::min(n_full, p.tiles);
}

bool sk_valid(const SkPlan& p) {
  const int64_t n_tail = p.tiles - p.n_full;
  return p.S > 1 && n_tail > 0 && n_tail <= kCounterBytes / 4 &&
         (int64_t)p.S * n_tail * p.bm * p.bn * 4 < ((int64_t)1 << 31);
}

// Tail plan for the large tile (256 x 256): split only the tiles of a last,
// partial round over the chip, e.g. 1152 tiles on 256 CUs run 1024 whole
// and split the other 128 in two.
bool tail_plan(int64_t M, int64_t N, int64_t K, SkPlan& p) {
  p.bm = 256; p.bn = 256; p.kst = 128;
  const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
  const int cus = device_cus();
  if (T < cus) return false;
  const int64_t n_full = (T / cus) * cus, n_tail = T - n_full;
  if (n_tail == 0 || 2 * n_tail > cus) return false;  // a tail of more than half a round runs fine whole
  const int S = (int)std::min<int64_t>(4, cus / n_tail);
  if ((K + 127) / 128 < 4 * S) return false;  // keep at least 4 stages per split
  sk_finish(p, M, N, K, S, (int)n_full);
  return sk_valid(p);
}

bool sk_plan(int64_t M, int64_t N, int64_t K, SkPlan& p) {
  if (sk_config(gemm_variant(), p)) {
    static const int S_env = [] {
      const char* e = getenv("FRT_GEMM_SPLITK");
      return e ? atoi(e) : 2;
    }();
    sk_finish(p, M, N, K, S_env, 0);
    return sk_valid(p);
  }
  // selectable only: measured slower than running the partial round whole
  // (8192 x 9216 x 3072: 246 -> 278 us; the split tiles' partial traffic
  // runs at the per-CU fill rate and their blocks lose L2 locality)
  if (gemm_variant() == 66 && M >= 512) return tail_plan(M, N, K, p);
  return false;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  SkPlan q{};
  if (sk_plan(M, N, K, q))
    return (size_t)(kCounterBytes + (int64_t)q.S * (q.tiles - q.n_full) * q.bm * q.bn * 4);
  if (!use_skinny(M, N)) return 0;
  const SkinnyPlan p = skinny_plan(M, N, K);
  if (p.splits <= 1) return 0;
  return (size_t)(kCounterBytes + (int64_t)p.splits * M * N * 4);
}

namespace {

template <int BM, int BN, int WM, int WN, int NSTAGE, int GM, bool PP>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  if (a.K % 64 == 0)
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WM, WN, NSTAGE, GM, PP, false>), dim3(tiles), dim3(threads),
                       0, st, a);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WM, WN, NSTAGE, GM, PP, true>), dim3(tiles), dim3(threads),
                       0, st, a);
  return hipGetLastError();
}

template <int MG, int NCH>
hipError_t launch_skinny_k(const GemmArgs& a, const SkinnyPlan& p, hipStream_t st) {
  const dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
  // the tail-free form needs every split's K range to lie inside K
  if (a.K % (128 * NCH) == 0)
    hipLaunchKernelGGL((gemm_skinny_kernel<MG, NCH, false>), grid, dim3(256), 0, st, a, p.splits);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<MG, NCH, true>), grid, dim3(256), 0, st, a, p.splits);
  return hipGetLastError();
}

template <int MG>
hipError_t launch_skinny_m(const GemmArgs& a, const SkinnyPlan& p, hipStream_t st) {
  switch (p.nch) {
    case 2: return launch_skinny_k<MG, 2>(a, p, st);
    case 4: return launch_skinny_k<MG, 4>(a, p, st);
    default: return launch_skinny_k<MG, 8>(a, p, st);
  }
}

hipError_t launch_skinny(const GemmArgs& a_in, hipStream_t st) {
  const SkinnyPlan p = skinny_plan(a_in.M, a_in.N, a_in.K);
  GemmArgs a = a_in;
  if (p.splits > 1) {  // counters first, then the partial planes
    a.cnt = reinterpret_cast<unsigned*>(a_in.ws);
    a.ws = reinterpret_cast<uint8_t*>(a_in.ws) + kCounterBytes;
  }
  switch (p.mg) {
    case 1: return launch_skinny_m<1>(a, p, st);
    case 2: return launch_skinny_m<2>(a, p, st);
    default: return launch_skinny_m<4>(a, p, st);
  }
}

template <int BM, int BN, int WM, int WN, int NS, int GM, int NSUB = 1>
hipError_t launch_big(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  if (a.K % (128 * NSUB) == 0)
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, WM, WN, NS, GM, false, NSUB>), dim3(tiles), dim3(threads), 0, st,
                       a);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, WM, WN, NS, GM, true, NSUB>), dim3(tiles), dim3(threads), 0, st,
                       a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NS, int GM>
hipError_t launch_k64(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  if (a.K % 64 == 0)
    hipLaunchKernelGGL((gemm_k64_kernel<BM, BN, WM, WN, NS, GM, false>), dim3(tiles), dim3(threads), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_k64_kernel<BM, BN, WM, WN, NS, GM, true>), dim3(tiles), dim3(threads), 0, st, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NS, int GM, int NSUB = 1>
hipError_t launch_big_sk(const GemmArgs& a_in, const SkPlan& p, hipStream_t st) {
  GemmArgs a = a_in;
  a.cnt = reinterpret_cast<unsigned*>(a_in.ws);
  a.ws = reinterpret_cast<uint8_t*>(a_in.ws) + kCounterBytes;
  a.kc = p.kc;
  a.nsplit = p.S;
  a.n_full = p.n_full;
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  const dim3 grid((unsigned)(p.n_full + (p.tiles - p.n_full) * p.S));
  if (a.K % (128 * NSUB) == 0)
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, WM, WN, NS, GM, false, NSUB, true>), grid, dim3(threads), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BM, BN, WM, WN, NS, GM, true, NSUB, true>), grid, dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  const int variant = gemm_variant();
  SkPlan sk{};
  if (sk_plan(a.M, a.N, a.K, sk)) {
    switch (variant) {
      case 60: return launch_big_sk<64, 64, 32, 32, 3, 1>(a, sk, st);
      case 61: return launch_big_sk<64, 32, 32, 32, 4, 1>(a, sk, st);
      case 62: return launch_big_sk<64, 128, 32, 64, 3, 1>(a, sk, st);
      case 63: return launch_big_sk<32, 64, 32, 32, 4, 1>(a, sk, st);
      case 64: return launch_big_sk<64, 32, 32, 32, 6, 1>(a, sk, st);
      case 65: return launch_big_sk<64, 64, 32, 32, 3, 1, 2>(a, sk, st);
      default: return launch_big_sk<256, 256, 128, 64, 2, 4>(a, sk, st);  // tail plan
    }
  }
  if (variant >= 10 && variant < 60) {  // tile-shape exploration
    switch (variant) {
      case 10: return launch_big<128, 64, 32, 32, 4, 2>(a, st);   // 8 waves
      case 11: return launch_big<128, 64, 32, 32, 6, 2>(a, st);
      case 12: return launch_big<64, 64, 32, 32, 4, 1>(a, st);    // 4 waves
      case 13: return launch_big<64, 64, 32, 32, 6, 1>(a, st);
      case 14: return launch_big<64, 32, 32, 32, 6, 1>(a, st);    // 2 waves
      case 15: return launch_big<32, 64, 32, 32, 6, 1>(a, st);    // 2 waves
      case 16: return launch_big<128, 128, 64, 32, 4, 2>(a, st);  // 8 waves
      case 17: return launch_big<256, 64, 64, 32, 4, 2>(a, st);   // 8 waves
      case 20: return launch_big<128, 64, 32, 32, 3, 2>(a, st);   // 8 waves, 72 KiB
      case 21: return launch_big<128, 128, 64, 32, 2, 2>(a, st);  // 8 waves, 64 KiB
      case 22: return launch_big<256, 64, 64, 32, 3, 2>(a, st);   // 8 waves, 120 KiB
      case 23: return launch_big<128, 64, 64, 32, 3, 2>(a, st);   // 4 waves, 72 KiB
      case 24: return launch_big<64, 64, 32, 32, 3, 1>(a, st);    // 4 waves, 48 KiB
      case 25: return launch_big<64, 32, 32, 32, 4, 1>(a, st);    // 2 waves, 48 KiB
      case 26: return launch_big<128, 32, 32, 32, 4, 2>(a, st);   // 4 waves, 80 KiB
      case 27: return launch_big<128, 128, 64, 32, 3, 2>(a, st);  // 8 waves, 96 KiB
      case 30: return launch_big<64, 32, 32, 32, 8, 1>(a, st);    // 2 waves, 96 KiB
      case 31: return launch_big<64, 32, 32, 32, 12, 1>(a, st);   // 2 waves, 144 KiB
      case 32: return launch_big<64, 64, 32, 32, 8, 1>(a, st);    // 4 waves, 128 KiB
      case 33: return launch_big<128, 64, 32, 32, 6, 2>(a, st);   // 8 waves, 144 KiB
      case 34: return launch_big<64, 32, 32, 32, 6, 1>(a, st);    // 2 waves, 72 KiB (2/CU)
      case 35: return launch_big<32, 64, 32, 32, 10, 1>(a, st);   // 2 waves, 120 KiB
      case 36: return launch_big<128, 32, 32, 32, 6, 2>(a, st);   // 4 waves, 120 KiB
      case 40: return launch_big<64, 64, 32, 32, 3, 1, 2>(a, st);   // 4 waves, K 256/stage, 96 KiB
      case 41: return launch_big<64, 64, 32, 32, 4, 1, 2>(a, st);   // 128 KiB
      case 42: return launch_big<64, 32, 32, 32, 4, 1, 2>(a, st);   // 2 waves, 96 KiB
      case 43: return launch_big<64, 32, 32, 32, 6, 1, 2>(a, st);   // 2 waves, 144 KiB
      case 44: return launch_big<128, 64, 32, 32, 3, 2, 2>(a, st);  // 8 waves, 144 KiB
      case 45: return launch_big<128, 64, 32, 32, 2, 2, 2>(a, st);  // 8 waves, 96 KiB
      case 46: return launch_big<32, 64, 32, 32, 4, 1, 2>(a, st);   // 2 waves, 96 KiB
      case 47: return launch_big<128, 128, 32, 32, 4, 2>(a, st);   // 16 waves, 128 KiB
      case 48: return launch_big<128, 128, 32, 32, 3, 2>(a, st);   // 16 waves, 96 KiB
      case 49: return launch_big<256, 128, 64, 64, 3, 4>(a, st);   // 8 waves, 144 KiB
      case 50: return launch_big<256, 128, 64, 32, 2, 4>(a, st);   // 16 waves, 96 KiB
      case 51: return launch_big<128, 256, 64, 64, 3, 2>(a, st);   // 8 waves, 144 KiB
      case 52: return launch_big<256, 256, 128, 128, 2, 4>(a, st);  // 4 waves, 128 KiB
      case 53: return launch_big<256, 128, 128, 64, 2, 4>(a, st);   // 4 waves, 96 KiB
      case 54: return launch_big<256, 256, 64, 128, 2, 4>(a, st);   // 8 waves, 128 KiB
      case 57: return launch_big<128, 256, 64, 64, 3, 2>(a, st);    // 8 waves, 144 KiB
      case 58: return launch_big<256, 128, 64, 64, 3, 4>(a, st);    // 8 waves, 144 KiB
      case 59: return launch_big<256, 128, 128, 64, 3, 4>(a, st);   // 4 waves, 144 KiB
      case 70: return launch_k64<256, 256, 128, 64, 4, 4>(a, st);   // 8 waves, 128 KiB
      case 71: return launch_k64<256, 256, 64, 128, 4, 4>(a, st);   // 8 waves, 128 KiB
      case 72: return launch_k64<256, 128, 64, 64, 6, 4>(a, st);    // 8 waves, 144 KiB
      case 73: return launch_k64<128, 256, 64, 64, 6, 2>(a, st);    // 8 waves, 144 KiB
      case 74: return launch_k64<128, 128, 64, 32, 8, 2>(a, st);    // 8 waves, 128 KiB
      case 75: return launch_k64<128, 128, 32, 32, 8, 2>(a, st);    // 16 waves, 128 KiB
      case 76: return launch_k64<64, 64, 32, 32, 8, 1>(a, st);      // 4 waves, 64 KiB
      case 77: return launch_k64<64, 32, 32, 32, 8, 1>(a, st);      // 2 waves, 48 KiB
      case 78: return launch_k64<256, 256, 128, 64, 2, 4>(a, st);   // 8 waves, 64 KiB
      default: break;
    }
  }
  if (use_skinny(a.M, a.N)) return launch_skinny(a, st);
  // Default plans (measured on MI355X, graph-replayed launches):
  //  M >= 512: 256x256 tiles, 8 waves of 128x64 (MFMA-bound shapes);
  //  64 < M < 512: 128x128 tiles of sixteen 32x32 waves when they fill the
  //    chip, else 64x64 tiles (more blocks for narrow N);
  //  M <= 64: 64x32 tiles, 256-deep K stages (weight streaming).
  if (a.M >= 512) return launch_big<256, 256, 128, 64, 2, 4>(a, st);
  if (a.M > 64) {
    if (((a.M + 127) / 128) * ((a.N + 127) / 128) >= 192) return launch_big<128, 128, 32, 32, 3, 2>(a, st);
    return launch_big<64, 64, 32, 32, 4, 1>(a, st);
  }
  return launch_big<64, 32, 32, 32, 4, 1, 2>(a, st);
}

}  // namespace frt
