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
// Tiles are staged through LDS with direct buffer->LDS loads, in 128-deep K
// stages (a stage may hold NSUB of them), row-major with one 128-byte
// segment per tile row and an XOR swizzle of its 16-byte chunks (see the
// kernel comment). An NS-deep ring keeps NS - 1 stages in flight; one block
// barrier per stage.
//
// Rows beyond M (or N) and K chunks beyond K read zeros: their buffer offset
// is pushed past the buffer's record count, which the hardware turns into a
// zero fill.
//
// Block order is XCD-aware: the dispatcher places block b on XCD b % 8, so
// the logical tile index gives each XCD a contiguous run of tiles, and runs
// are rastered in groups of GM tile-rows so that the tiles resident on one
// XCD share A and B panels in that XCD's L2.
#include <cstdint>
#include <type_traits>
#include <utility>

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

// s_waitcnt immediate: vmcnt(n) together with lgkmcnt(0) (expcnt left at its
// maximum)
__device__ __forceinline__ constexpr int vm_lgkm0_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4);
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


// Tiled kernel: BM x BN block tile, WM x WN per wave, 128-deep K staging.
//
// LDS holds each stage row-major, one 128-byte row segment per tile row, with
// the eight 16-byte chunks of row r stored at chunk position
// c ^ ((r >> 1) & 7) (an XOR swizzle). A direct buffer->LDS load
// instruction of a wave therefore covers 8 rows x 128 contiguous bytes (whole
// cache lines), and each lane's destination stays lane-contiguous as the
// instruction requires: lane L writes chunk position L % 8 of row L / 8, so
// it fetches global chunk (L % 8) ^ ((row >> 1) & 7). A 32x32x64 operand
// read (row l % 32, K bytes [s*64 + (l/32)*32, +32)) takes chunks
// c0 = s*4 + (l/32)*2 and c0 + 1, i.e. positions c0 ^ ((l >> 1) & 7) and
// that ^ 1. The LDS serves a ds_read_b128 sixteen lanes (256 bytes, all 64
// banks) at a time: sixteen consecutive rows fall in two 128-byte halves by
// row parity and on eight distinct positions within each half, so the reads
// are conflict free.
//
// A stage holds NSUB such 128-deep sub-buffers; an NS-deep ring keeps the
// loads of NS - 1 stages in flight, with one block barrier per stage, after
// which the slot read two barriers earlier is refilled. Small wave tiles
// read all of a stage's operand fragments right after the barrier and
// alternate between two accumulator sets (independent MFMAs back to back);
// large wave tiles (two waves per SIMD) reuse one fragment set and rely on
// the other wave of the SIMD to cover the fragment reads.
// AE (<= BM): A rows actually loaded. A call with M <= AE leaves tile rows
// [AE, BM) unloaded: their MFMA results only reach output rows >= M, which
// the epilogue never stores, and every wave still issues the same number of
// loads per stage, so the vmcnt counts stay exact.
//
// GLU: the gate/up GEGLU form. W8 holds 2H rows (gate rows, then up rows)
// and a tile covers BN/2 gate columns [g0, g0 + BN/2) together with the
// matching up columns: tile-local B row r is gate row g0 + (r/64)*32 + r%32
// when (r/32) is even and the up row H + (the same) when it is odd. A
// 64-column wave tile therefore holds gate column c in accumulator pair
// 2q and up column c in 2q + 1 of the same lane, and the epilogue writes
// e4m3(gelu_tanh(bf16(gate)) * bf16(up) / q_scale) for H columns. Gate rows
// past H (a ragged last tile) read up rows, whose results are never stored;
// up rows past 2H read zeros. With FP4 the same rows are loaded (K/2 bytes
// a row) and each lane takes the block scales of the row it multiplies.
//
// ROPE: the QKV split + RoPE + KV-cache form. Columns [0, nh hd) are q,
// the next kv hd are k, the last kv hd are v, with the q and k rows
// pair-interleaved at pack time so that each rotary pair is two adjacent
// columns, i.e. lanes l and l ^ 1 of the MFMA layout: each lane rounds its
// value to bf16 as the split output would be, takes its partner's through
// DPP, rotates q and k with the pair's (cos, sin) from the token's rope row,
// and writes q_out row m, or cache row P + m of k or v.
//
// FP4: the MXFP4 form. x and W hold e2m1 codes, two per byte (K/2 bytes a
// row), with one E8M0 scale per 32 K-elements in sa [M, ld_sa] and sb
// [N, K/32]. A 128-byte stage row holds 256 K-elements, i.e. four 64-deep
// MFMA steps, each reading one 16-byte chunk per operand (lane l: row l % 32,
// K half l / 32 = exactly one scale block). The scales are stored run-major,
// [K/256][rows][8] (run stride ld_sa for x, 8 N for W), each run of 8 blocks
// (256 K-elements) in the order 0, 2, 4, 6, 1, 3, 5, 7: the lanes of K half
// h take one dword holding their blocks h, 2 + h, 4 + h, 6 + h (a 32-row
// block's dwords for one run are 256 contiguous bytes) and step s selects
// byte s. Each run's scales of the tile's rows are staged in LDS beside the
// tiles: one direct dword load per 32-row block (A rows, then the B rows in
// tile order), issued by the same call as the tiles and spread over the
// waves (the wait counts cover them), and read back with the fragments, so
// a block's scales are fetched once, not once per wave that uses them. Rows
// past M or N fetch zeros (each run has its own record count); their results
// are never stored. alpha is 1.
template <int BM, int BN, int WM, int WN, int NS, int GM, bool KTAIL, int NSUB, int AE = BM,
          bool GLU = false, bool ROPE = false, bool FP4 = false>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(GemmArgs a) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NW = (BM / WM) * WAVES_N;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int ROWS = BM + BN;
  static_assert(AE <= BM && AE % 16 == 0, "A rows loaded");
  static_assert(!GLU || (NJ % 2 == 0 && WN % 64 == 0), "GEGLU pairs need 64-column wave tiles");
  constexpr int LOADS = (AE + BN) / 8;  // 1 KiB load instructions per stage
  static_assert(LOADS % NW == 0, "loads must split evenly over the waves");
  constexpr int LPW = LOADS / NW;
  constexpr int SUBB = ROWS * 128;     // one 128-deep sub-buffer
  constexpr int STAGE = NSUB * SUBB;   // one stage = NSUB sub-buffers
  constexpr int KST = 128 * NSUB;      // K bytes per stage
  static_assert(!FP4 || !KTAIL, "MXFP4 form: whole stages");
  // MXFP4 scale staging: AER A rows (AE rounded up to 32) and BN B rows of
  // 8 bytes per run, SLT 32-row loads per sub-buffer; every wave issues SCL
  // of them, wave w load k being block min(w + k NW, SLT - 1) (a repeated
  // block writes the same bytes to the same place)
  constexpr int AER = (AE + 31) / 32 * 32;
  constexpr int SLT = FP4 ? AER / 32 + BN / 32 : 0;
  constexpr int SCB = FP4 ? (AER + BN) * 8 : 0;  // scale bytes per sub-buffer
  constexpr int SCL = (SLT + NW - 1) / NW;
  static_assert(BN % 32 == 0, "32-row scale loads");
  static_assert(NS >= 2 && NSUB * (LPW + SCL) * (NS - 2) <= 63, "ring depth vs vmcnt range");
  constexpr int SCBASE = NS * STAGE;  // the scale area follows the ring
  static_assert(NS * (STAGE + NSUB * SCB) <= 160 * 1024, "ring exceeds LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * (STAGE + NSUB * SCB)];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const TileXY t = tile_of(blockIdx.x, tiles_m, tiles_n, GM);
  // n0: first output column (GLU: first gate column g0)
  const int m0 = t.tm * BM, n0 = t.tn * (GLU ? BN / 2 : BN);
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

  const int Kb = FP4 ? a.K / 2 : a.K;  // operand bytes per row
  const uint32_t x_bytes = (uint32_t)((int64_t)(a.M - 1) * a.ld_x + Kb);
  const uint32_t w_bytes = (uint32_t)((int64_t)a.N * Kb);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, w_bytes);

  // this wave's load instructions: tile rows [8u, 8u + 8), u = wave + j*NW.
  // One base offset per operand; instruction j adds a uniform multiple of
  // the row stride. A row past M (N) lands past the buffer's record count
  // ((M-1)*ld_x + K, resp. N*K, with ld_x >= K), which the hardware turns
  // into a zero fill, so no per-load bound registers are kept.
  static_assert(AE % (8 * NW) == 0 && BN % (8 * NW) == 0, "A and B loads split evenly");
  constexpr int LPA = AE / (8 * NW);  // the first LPA loads of a wave are A rows
  const int lrow = lane >> 3;
  // global chunk this lane fetches: rows 8u + lrow with u = wave + j*NW and
  // NW even, so (row >> 1) & 7 = ((wave & 1) << 2) | (lrow >> 1) for every j
  static_assert(NW % 2 == 0, "row swizzle assumes an even wave count");
  const int cch = (lane & 7) ^ (((wave & 1) << 2) | (lrow >> 1));
  const uint32_t offA = (uint32_t)((int64_t)(m0 + wave * 8 + lrow) * a.ld_x) + cch * 16;
  const uint32_t offB = GLU ? (uint32_t)(lrow * Kb + cch * 16)
                            : (uint32_t)((int64_t)(n0 + wave * 8 + lrow) * Kb) + cch * 16;
  const uint32_t stepA = (uint32_t)(8 * NW) * (uint32_t)a.ld_x;
  const uint32_t stepB = (uint32_t)(8 * NW) * (uint32_t)Kb;
  const int KT = (Kb + KST - 1) / KST;
  // MXFP4 scales of the stage being multiplied, read from LDS with the
  // fragments: sub-buffer q, this lane's A (B) row block i (j)
  unsigned sA[FP4 ? NSUB : 1][FP4 ? MI : 1], sB[FP4 ? NSUB : 1][FP4 ? NJ : 1];
  // this wave's scale loads, chosen once by uniform selects: source buffer,
  // run stride, per-run record count, byte offset of the block's first row
  // and LDS offset; under GLU B block g is gate (g even) or up rows of the
  // 32-column pair g / 2
  constexpr int SCK = FP4 ? SCL : 1;
  const uint8_t* sc_src[SCK];
  int64_t sc_run[SCK];
  uint32_t sc_rec[SCK], sc_off[SCK], sc_lds[SCK];
  // a block lands K-half-major (LDS dword l holds row l % 32, half l / 32),
  // so the lanes of the MFMA layout read consecutive dwords
  const uint32_t sc_lane = (uint32_t)((lane & 31) * 8 + (lane >> 5) * 4);
  if constexpr (FP4) {
#pragma unroll
    for (int k = 0; k < SCL; ++k) {
      const int s = min(wave + k * NW, SLT - 1);
      const bool isA = s < AER / 32;
      const int g = s - AER / 32;
      const int row = isA ? m0 + s * 32 : GLU ? (g & 1) * a.H + n0 + (g >> 1) * 32 : n0 + g * 32;
      sc_src[k] = isA ? a.sa : a.sb;
      sc_run[k] = isA ? a.ld_sa : (int64_t)a.N * 8;
      sc_rec[k] = (uint32_t)(isA ? a.M : a.N) * 8u;
      sc_off[k] = (uint32_t)row * 8u;
      sc_lds[k] = isA ? s * 256 : AER * 8 + g * 256;
    }
  }
  // slot SL (= step mod NS) is a compile-time constant in every use, so all
  // LDS addresses are one lane base plus immediates
  auto issue = [&](int kt, auto SLC) {
    constexpr int SL = decltype(SLC)::value;
#pragma unroll
    for (int q = 0; q < NSUB; ++q) {
      const int k0 = kt * KST + q * 128;
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const bool A = j < LPA;
        // A rows 8u.., B rows BM + 8u.. (u counts this operand's loads)
        const int u = wave + (A ? j : j - LPA) * NW + (A ? 0 : BM / 8);
        uint8_t* dst = smem + SL * STAGE + q * SUBB + u * 1024;
        uint32_t o;
        if (A) {
          o = offA + j * stepA + k0;
        } else if constexpr (GLU) {
          // B unit ub (tile-local rows 8ub .. 8ub + 7): gate or up half by
          // (ub / 4) % 2, 32-column pair ub / 8, 8-row group ub % 4
          const int ub = wave + (j - LPA) * NW;
          const int row = ((ub >> 2) & 1) * a.H + n0 + (ub >> 3) * 32 + (ub & 3) * 8;
          o = offB + (uint32_t)row * (uint32_t)Kb + k0;
        } else {
          o = offB + (j - LPA) * stepB + k0;
        }
        if constexpr (KTAIL) {
          if (k0 + cch * 16 >= a.K) o = kOOB;
        }
        if (A)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
      }
      if constexpr (FP4) {
        // the scales of run kt * NSUB + q: 32 rows (256 bytes) per load
        const int64_t run = kt * NSUB + q;
        uint8_t* sdst = smem + SCBASE + (SL * NSUB + q) * SCB;
#pragma unroll
        for (int k = 0; k < SCL; ++k) {
          const __amdgpu_buffer_rsrc_t r = make_rsrc(sc_src[k] + run * sc_run[k], sc_rec[k]);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(sdst + sc_lds[k]), 4, sc_lane, sc_off[k], 0, 0);
        }
      }
    }
  };
  // operand read of substep SUB from slot SL: two 16-byte chunks per lane
  const int lrow32 = lane & 31;
  const int sw = (lrow32 >> 1) & 7;  // (row >> 1) & 7 for rows 32k + lrow32
  const uint8_t* lbase0 = smem + lrow32 * 128 + ((((lane >> 5) * 2) ^ sw) * 16);
  const uint8_t* lbase1 = smem + lrow32 * 128 + ((((lane >> 5) * 2 + 4) ^ sw) * 16);
  // this lane's scale dword within a 32-row block: row lrow32, K half l / 32
  const uint8_t* sbase = smem + SCBASE + lane * 4;
  auto read_frags = [&](auto SLC, auto SUBC, auto* af, auto* bf) {
    constexpr int SL = decltype(SLC)::value, SUB = decltype(SUBC)::value;
    if constexpr (FP4) {
      // step SUB % 4 of sub-buffer SUB / 4: chunk 2 (SUB % 4) + l / 32
      const uint8_t* lb = smem + lrow32 * 128 + ((((SUB & 3) * 2 + (lane >> 5)) ^ sw) * 16) + SL * STAGE +
                          (SUB >> 2) * SUBB;
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *reinterpret_cast<const v4i*>(lb + (BM + wn0 + j * 32) * 128);
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = *reinterpret_cast<const v4i*>(lb + (wm0 + i * 32) * 128);
      if constexpr ((SUB & 3) == 0) {
        // the sub-buffer's scales; A blocks past the AER staged rows (rows
        // past M) take the last staged block
        constexpr int Q = SUB >> 2;
        const uint8_t* sp = sbase + (SL * NSUB + Q) * SCB;
#pragma unroll
        for (int i = 0; i < MI; ++i)
          sA[Q][i] = *reinterpret_cast<const unsigned*>(sp + min(wm0 + i * 32, AER - 32) * 8);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          sB[Q][j] = *reinterpret_cast<const unsigned*>(sp + (AER + wn0 + j * 32) * 8);
      }
      return;
    } else {
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
    }
  };
  // own loads: at most `ahead` later stages still in flight; every LDS read
  // done; then the block barrier (s_waitcnt takes an immediate: one case per
  // possible depth)
  auto sync_stage = [&](int ahead) {
    __builtin_amdgcn_sched_barrier(0);
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((ahead == I ? (__builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(NSUB * (LPW + SCL) * I)), 0) : 0), ...);
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
  constexpr int KSUB = (FP4 ? 4 : 2) * NSUB;
  constexpr bool ALL = MI * NJ * KSUB <= 8;
  constexpr int NACC = (ALL && KSUB >= 2) ? 2 : 1;
  constexpr int NF = ALL ? KSUB : 1;
  // (FP4 fragments use the low four dwords only; the MFMA reads four
  // registers per operand for e2m1)
  typedef std::conditional_t<FP4, v4i, v8i> frag_t;
  frag_t fa[NF][MI], fb[NF][NJ];
  v16f acc2[NACC > 1 ? MI : 1][NACC > 1 ? NJ : 1];
  if constexpr (NACC > 1) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc2[i][j][r] = 0.0f;
  }
  auto mfmas = [&](const frag_t* af, const frag_t* bf, auto ACC, auto SLC, auto SUBC) {
    constexpr int SUB = decltype(SUBC)::value;
#pragma unroll
    for (int q = 0; q < MI * NJ; ++q) {
      const int i = q / NJ, j = q % NJ;
      v16f& c = decltype(ACC)::value == 0 ? acc[i][j] : acc2[NACC > 1 ? i : 0][NACC > 1 ? j : 0];
      if constexpr (FP4) {
        // step s of the sub-buffer: byte s of the lane's scale dword
        constexpr int s = SUB & 3, sb = SUB >> 2;
        const v8i a8 = {af[i][0], af[i][1], af[i][2], af[i][3], 0, 0, 0, 0};
        const v8i b8 = {bf[j][0], bf[j][1], bf[j][2], bf[j][3], 0, 0, 0, 0};
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, s, (int)sA[sb][i], s,
                                                           (int)sB[sb][j]);
      } else {
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], c, 0, 0, 0, 0, 0, 0);
      }
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
        (mfmas(fa[U], fb[U], std::integral_constant<int, U % NACC>{}, SLC, std::integral_constant<int, U>{}), ...);
      }(std::make_integer_sequence<int, KSUB>{});
    } else {
      [&]<int... U>(std::integer_sequence<int, U...>) {
        ((U > 0 ? (read_frags(SLC, std::integral_constant<int, U>{}, fa[0], fb[0]), 0) : 0,
          mfmas(fa[0], fb[0], std::integral_constant<int, 0>{}, SLC, std::integral_constant<int, U>{})), ...);
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

  // ---- epilogue: alpha * acc + bias, column split, bf16 (or fp32) ----
  const float alpha = FP4 ? 1.0f : (*a.act_scale) * (*a.w_scale);
  if constexpr (ROPE) {
    const int nq = a.nh * a.hd, nk = a.kv * a.hd;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn0 + j * 32 + (lane & 31);
      const bool nok = n < a.N;
      const bool rot = n < nq + nk;
      const int d = n % a.hd;
      const float b = (a.bias != nullptr && nok) ? bf16f(a.bias[n]) : 0.0f;
      uint16_t* dst;
      int64_t ld;
      if (n < nq) {
        dst = a.q_out + n;
        ld = nq;
      } else if (rot) {
        dst = a.k_cache + a.P * nk + (n - nq);
        ld = nk;
      } else {
        dst = a.v_cache + a.P * nk + (n - nq - nk);
        ld = nk;
      }
      // a' = a c - b s on the even column, b' = b c + a s on the odd one
      const float sgn = (n & 1) ? 1.0f : -1.0f;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        // the (cos, sin) words of this lane's 16 rows, loaded together (rows
        // past M read row M - 1 and are not stored)
        uint32_t cs[16];
        const uint16_t* rp = a.rope + (d & ~1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = min(m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3), a.M - 1);
          cs[r] = rot ? *reinterpret_cast<const uint32_t*>(rp + (int64_t)m * a.hd) : 0u;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const float v = __uint_as_float(f2bf(alpha * acc[i][j][r] + b) << 16);
          const float p = lane_xor1(v);
          const float o = rot ? __builtin_fmaf(v, bf16lo(cs[r]), sgn * (p * bf16hi(cs[r]))) : v;
          if (nok && m < a.M) dst[(int64_t)m * ld] = (uint16_t)f2bf(o);
        }
      }
    }
    return;
  }
  if constexpr (GLU) {
    if (a.q4 != nullptr) {
      // GEGLU to MXFP4: a block scale needs the maximum over 32 consecutive
      // columns, which the MFMA layout spreads over 32 lanes, so the wave's
      // y tile goes through LDS and comes back row-wise: 8 consecutive
      // columns per lane, one 32-column block per quad, quantised as the
      // standalone GEGLU -> MXFP4 kernel quantises them. The tiles go to
      // ring slot KT % NS, whose last stage (KT - NS) every wave finished
      // reading before a later barrier, when they fit in it; else to the
      // whole ring after a barrier. Each wave reads back only what it wrote.
      static_assert(NJ == 2, "one 32-column gate block per wave");
      constexpr int YR = MI * 32;  // rows of the wave's y tile (32 columns)
      constexpr bool ONE_SLOT = NW * YR * 32 * 4 <= STAGE;
      uint8_t* ybase = smem;
      if constexpr (ONE_SLOT)
        ybase = smem + (KT % NS) * STAGE;
      else
        __syncthreads();
      float* ys = reinterpret_cast<float*>(ybase) + wave * YR * 32;
      const int gc0 = n0 + (wn0 >> 1);  // the wave's first gate column
      const float bg = (a.bias != nullptr && gc0 < a.H) ? bf16f(a.bias[gc0 + (lane & 31)]) : 0.0f;
      const float bu = (a.bias != nullptr && gc0 < a.H) ? bf16f(a.bias[a.H + gc0 + (lane & 31)]) : 0.0f;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const float vg = alpha * acc[i][0][r] + bg;
          const float vu = alpha * acc[i][1][r] + bu;
          ys[rl * 32 + (lane & 31)] =
              gelu_tanh(__uint_as_float(f2bf(vg) << 16)) * __uint_as_float(f2bf(vu) << 16);
        }
      }
      __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(63));  // this wave's LDS writes done
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < YR * 4 / 64; ++k) {
        const int t = lane + 64 * k, rl = t >> 2, v = t & 3;
        const float4 y0 = *reinterpret_cast<const float4*>(ys + rl * 32 + v * 8);
        const float4 y1 = *reinterpret_cast<const float4*>(ys + rl * 32 + v * 8 + 4);
        const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) am = max(am, __float_as_uint(fabsf(y[e])));
        const uint32_t sbyte = e8m0_of_amax(quad_umax(am));
        const uint32_t codes = mxfp4_pack8(y, sbyte);
        const int m = m0 + wm0 + rl;
        if (m < a.M && gc0 < a.H) {
          const int64_t c = gc0 + v * 8;
          *reinterpret_cast<uint32_t*>(a.q4 + (int64_t)m * a.ld_q4 + c / 2) = codes;
          if (v == 0) a.sc4[e8m0_off(m, c / 32, a.ld_sc4)] = (uint8_t)sbyte;
        }
      }
      return;
    }
    // gate and up rounded to bf16 as the unfused GEMM output would be,
    // then the GEGLU quantiser of frt_ffn.hip
    const float qs = *a.q_scale, qr = 1.0f / qs;
#pragma unroll
    for (int q = 0; q < NJ / 2; ++q) {
      const int gc = n0 + (wn0 >> 1) + q * 32 + (lane & 31);
      if (gc >= a.H) continue;
      const float bg = a.bias != nullptr ? bf16f(a.bias[gc]) : 0.0f;
      const float bu = a.bias != nullptr ? bf16f(a.bias[a.H + gc]) : 0.0f;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          if (m < a.M) {
            const float vg = alpha * acc[i][2 * q][r] + bg;
            const float vu = alpha * acc[i][2 * q + 1][r] + bu;
            const float y = gelu_tanh(__uint_as_float(f2bf(vg) << 16)) * __uint_as_float(f2bf(vu) << 16);
            a.q8[(int64_t)m * a.ld_q8 + gc] = (uint8_t)cvt2_fp8(clamp_fp8(div_rn(y, qs, qr)), 0.0f);
          }
        }
      }
    }
    return;
  }
  // Waves of 128 x 64 (the 256x256 plan) hold whole 128-byte row segments
  // of the bf16 output. With vec_out they pass them through LDS, 64 rows at
  // a time, and store 16 bytes a lane (8 rows x 128 bytes an instruction)
  // instead of the 64-byte halves the MFMA layout gives. Each wave uses its
  // own 8 KB of ring slot KT % NS, whose last stage every wave finished
  // reading before an earlier barrier and into which no load is pending, so
  // no block barrier is needed. Within the 64 x 128-byte buffer, 16-byte
  // chunk c of row r sits at position c ^ (r & 7).
  constexpr bool WIDE = !GLU && !ROPE && !FP4 && WN == 64 && NJ == 2 && MI % 2 == 0 &&
                        NW * 64 * 128 <= STAGE;
  if constexpr (WIDE) {
    if (a.vec_out) {
      uint8_t* wb = smem + (KT % NS) * STAGE + wave * (64 * 128);
      float bj[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn0 + j * 32 + (lane & 31);
        bj[j] = (a.bias != nullptr && n < a.N) ? bf16f(a.bias[n]) : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < MI / 2; ++h) {
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rr = i2 * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);  // row in the half
              const int c = j * 32 + (lane & 31);                                  // column in the wave
              const float v = alpha * acc[2 * h + i2][j][r] + bj[j];
              *reinterpret_cast<uint16_t*>(wb + rr * 128 + (((c >> 3) ^ (rr & 7)) << 4) + (c & 7) * 2) =
                  (uint16_t)f2bf(v);
            }
        __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(63));
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int t = lane + 64 * k;
          const int rr = t >> 3, cc = t & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(wb + rr * 128 + ((cc ^ (rr & 7)) << 4));
          const int m = m0 + wm0 + h * 64 + rr;
          const int n = n0 + wn0 + cc * 8;
          if (m < a.M && n < a.N) {
            // split widths are multiples of 8: the chunk lies in one split
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
            *reinterpret_cast<uint4*>(base + ((int64_t)m * ld + (n - off0)) * 2) = v;
          }
        }
        __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(63));
        __builtin_amdgcn_wave_barrier();
      }
      return;
    }
  }
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

template <int BM, int BN, int WM, int WN, int NS, int GM, int NSUB = 1, int AE = BM, bool GLU = false,
          bool ROPE = false, bool FP4 = false>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t st) {
  // (GLU: N = 2H, so this is also ceil(H / (BN / 2)) column tiles)
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  if constexpr (FP4) {  // whole stages (K a multiple of 256 * NSUB) is checked by the caller
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, GM, false, NSUB, AE, GLU, ROPE, true>), dim3(tiles),
                       dim3(threads), 0, st, a);
    return hipGetLastError();
  }
  if (a.K % (128 * NSUB) == 0)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, GM, false, NSUB, AE, GLU, ROPE>), dim3(tiles),
                       dim3(threads), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, GM, true, NSUB, AE, GLU, ROPE>), dim3(tiles),
                       dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// The current plans use no workspace (the argument is kept in the ABI).
size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                   ? n
                   : 256;
  }
  return cus[dev];
}

// Operand bytes (per K byte) that the busiest CU loads under a BM x BN tile
// plan: tiles are dealt one per CU per round, and a tile loads BM + BN rows
// of K bytes. The per-CU fill rate bounds these kernels, so among plans the
// one with the smallest figure wins. Ties go to the smaller tile: at equal
// per-CU load it keeps more CUs busy (1024 x 8192 over K = 2048: 31.6 us
// for the 512 tiles of 128x128 against 39.6 us for the 128 tiles of
// 256x256; the GEGLU form 31.3 against 41.0 us; 256 x 8192: 14.6 us for
// 64x64 against 15.1 us for 128x128).
int64_t plan_cost(const GemmArgs& a, int BM, int BN, int cus) {
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  return ((tiles + cus - 1) / cus) * (BM + BN);
}

// Tile plans (measured on MI355X, graph-replayed launches with HBM-resident
// weights):
//  M > 64: the plan of least per-CU load (plan_cost) among 256x256 tiles of
//    eight 128x64 waves (M >= 512 only: the MFMA-bound shapes), 128x128 of
//    sixteen 32x32 waves, 64x64 of four 32x32 waves and 64x32 with 256-deep
//    stages. E.g. 256 x 16384 -> 128x128; 256 x 2560 -> 64x64 (160 tiles);
//    256 x 2048 over K = 8192 -> 64x32 (256 tiles: 17 us against 22 us for
//    the 128 tiles of 64x64);
//  M <= 64: 64x32 tiles with 256-deep stages (weight streaming), loading
//    only the first 16 or 32 A rows when M is at most that.
template <bool ROPE>
hipError_t launch_planned(const GemmArgs& a, hipStream_t st) {
  if (a.M > 64) {
    const int cus = device_cus();
    int best = 0;
    int64_t c = INT64_MAX;
    const int64_t cost[4] = {a.M >= 512 ? plan_cost(a, 256, 256, cus) : INT64_MAX, plan_cost(a, 128, 128, cus),
                             plan_cost(a, 64, 64, cus), plan_cost(a, 64, 32, cus)};
    for (int p = 0; p < 4; ++p)  // ordered large to small: ties go to the smaller tile
      if (cost[p] <= c) c = cost[p], best = p;
    switch (best) {
      case 0: return launch_tiles<256, 256, 128, 64, 2, 4, 1, 256, false, ROPE>(a, st);
      case 1: return launch_tiles<128, 128, 32, 32, 3, 2, 1, 128, false, ROPE>(a, st);
      case 2: return launch_tiles<64, 64, 32, 32, 4, 1, 1, 64, false, ROPE>(a, st);
      default: return launch_tiles<64, 32, 32, 32, 4, 1, 2, 64, false, ROPE>(a, st);
    }
  }
  // rows past M are not loaded (at M <= 16, 8 of every 12 load
  // instructions would only fetch zeros): M = 1 9.3 -> 8.8 us, M = 16
  // 9.8 -> 9.3 us for 6144 x 4096 weights. At M <= 16 a three-deep ring of
  // 512-deep stages keeps more of the weight stream in flight (M = 1
  // 8.75 -> 8.50 us, M = 16 9.23 -> 9.05 us; it loses at M = 32 and 64)
  if (a.M <= 16 && a.K % 512 == 0) return launch_tiles<64, 32, 32, 32, 3, 1, 4, 16, false, ROPE>(a, st);
  if (a.M <= 16) return launch_tiles<64, 32, 32, 32, 4, 1, 2, 16, false, ROPE>(a, st);
  if (a.M <= 32) return launch_tiles<64, 32, 32, 32, 4, 1, 2, 32, false, ROPE>(a, st);
  return launch_tiles<64, 32, 32, 32, 4, 1, 2, 64, false, ROPE>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) { return launch_planned<false>(a, st); }

// The RoPE epilogue runs on the split plans (any tile keeps a rotary pair in
// adjacent lanes).
hipError_t launch_gemm_rope(const GemmArgs& a, hipStream_t st) { return launch_planned<true>(a, st); }

// MXFP4 plans (K % 256 == 0: whole 256-element stages): the small-M plan
// for M <= 64; above, the least per-CU load among 128x128 of eight 32x64
// waves, 64x64 and 64x32. Half the bytes per row as FP8 move the balance
// toward larger tiles only through plan_cost's row counts. The 64x32 plans
// stage 1024 K-elements (four runs) in a three-deep ring when K allows it
// (6144 x 4096 weights: M = 1 7.7 -> 6.9 us, M = 16 8.2 -> 7.3 us, M = 64
// level), else 512 in a four-deep ring, else one run in a seven-deep ring.
template <int AE, bool ROPE>
hipError_t launch_mx_narrow(const GemmArgs& a, hipStream_t st) {
  if (a.K % 1024 == 0) return launch_tiles<64, 32, 32, 32, 3, 1, 4, AE, false, ROPE, true>(a, st);
  if (a.K % 512 == 0) return launch_tiles<64, 32, 32, 32, 4, 1, 2, AE, false, ROPE, true>(a, st);
  return launch_tiles<64, 32, 32, 32, 7, 1, 1, AE, false, ROPE, true>(a, st);
}

// The split plans; the RoPE form (the QKV split + RoPE + KV-cache epilogue)
// runs on the same tiles, so its results equal the split GEMM's bf16 output
// passed through the standalone consumer.
template <bool ROPE>
hipError_t launch_mx_planned(const GemmArgs& a, hipStream_t st) {
  if (a.M > 64) {
    const int cus = device_cus();
    const int64_t c128 = plan_cost(a, 128, 128, cus), c64 = plan_cost(a, 64, 64, cus),
                  c32 = plan_cost(a, 64, 32, cus);
    if (c128 < c64 && c128 < c32) return launch_tiles<128, 128, 32, 64, 3, 2, 1, 128, false, ROPE, true>(a, st);
    if (c64 < c32) return launch_tiles<64, 64, 32, 32, 4, 1, 1, 64, false, ROPE, true>(a, st);
    return launch_mx_narrow<64, ROPE>(a, st);
  }
  if (a.M <= 16) return launch_mx_narrow<16, ROPE>(a, st);
  if (a.M <= 32) return launch_mx_narrow<32, ROPE>(a, st);
  return launch_mx_narrow<64, ROPE>(a, st);
}

hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t st) { return launch_mx_planned<false>(a, st); }
hipError_t launch_gemm_mxfp4_rope(const GemmArgs& a, hipStream_t st) { return launch_mx_planned<true>(a, st); }

// MXFP4 GEGLU plans: the MXFP4 128x128 plan (its waves are already 32x64)
// where it has the least per-CU load, else 64x64 of two 32x64 waves; like
// the split plans they alternate two accumulator sets over the 64-deep
// steps, so the fused codes equal the split GEMM's bf16 output quantised by
// the standalone GEGLU kernel.
hipError_t launch_gemm_mxfp4_geglu(const GemmArgs& a, hipStream_t st) {
  if (a.M > 64) {
    const int cus = device_cus();
    if (plan_cost(a, 128, 128, cus) < plan_cost(a, 64, 64, cus))
      return launch_tiles<128, 128, 32, 64, 3, 2, 1, 128, true, false, true>(a, st);
  }
  return launch_tiles<64, 64, 32, 64, 4, 1, 1, 64, true, false, true>(a, st);
}

// GEGLU plans: the same tiles with 64-column wave tiles (a gate/up pair per
// lane), chosen by plan_cost: 256x256 (M >= 512), 128x128 of eight 32x64
// waves, 64x64 of two 32x64 waves (also every M <= 64).
hipError_t launch_gemm_geglu(const GemmArgs& a, hipStream_t st) {
  if (a.M > 64) {
    const int cus = device_cus();
    const int64_t c256 = a.M >= 512 ? plan_cost(a, 256, 256, cus) : INT64_MAX;
    const int64_t c128 = plan_cost(a, 128, 128, cus), c64 = plan_cost(a, 64, 64, cus);
    if (c256 < c128 && c256 < c64) return launch_tiles<256, 256, 128, 64, 2, 4, 1, 256, true>(a, st);
    if (c128 < c64) return launch_tiles<128, 128, 32, 64, 3, 2, 1, 128, true>(a, st);
  }
  return launch_tiles<64, 64, 32, 64, 4, 1, 1, 64, true>(a, st);
}

}  // namespace frt
