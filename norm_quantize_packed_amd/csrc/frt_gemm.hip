// Packed FP8 GEMM with dequant + bias + column-split epilogue on gfx950.
//
// out[m, n] = bf16(fl32(alpha * sum_k x8[m,k] * W8[n,k]) + bias[n]) written
// into the split s that owns column n (flashrt-structures 0.2.0,
// impls/qkv_pack/fp8_static.py `PackedLinear._run`; alpha = act_scale *
// w_scale as folded in impls/adarms_stack/fp8_chain.py `_quantize`).
//
// Both operands are K-contiguous ("TN"). The main loop runs on the CDNA4
// FP8 matrix cores, v_mfma_f32_32x32x64_f8f6f4 (A = 32 rows of x8, B = 32
// rows of W8, 64-deep K step, fp32 accumulate) in the tile kernels, and
// v_mfma_f32_16x16x128_f8f6f4 (16 rows each, 128-deep) in the 256 x 256
// kernel.
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
#include <atomic>
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
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr uint32_t kOOB = 0x80000000u;  // offset past any record count

// a byte in global memory (so stores through it are global, not flat)
typedef __attribute__((address_space(1))) uint8_t gbyte_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // flags: default data format for raw buffer loads on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt immediate: vmcnt(n) together with lgkmcnt(0) (expcnt left at its
// maximum)
__device__ __forceinline__ constexpr int vm_lgkm0_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4);
}

// s_waitcnt immediate: vmcnt(n) alone (lgkmcnt and expcnt at their maxima)
__device__ __forceinline__ constexpr int vm_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// s_waitcnt immediate: lgkmcnt(n) alone (vmcnt and expcnt at their maxima)
__device__ __forceinline__ constexpr int lgkm_imm(int n) {
  return 0xF | (0x3 << 14) | (0x7 << 4) | ((n & 0xF) << 8);
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
// AE (<= BM): A rows actually loaded, and the A rows a stage holds in LDS
// (the B rows follow them). A call with M <= AE needs no tile rows past AE:
// fragment reads of those rows take row 0 instead (in-bounds reads whose
// MFMA results only reach output rows >= M, which the epilogue never
// stores), and every wave still issues the same number of loads per stage,
// so the vmcnt counts stay exact.
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
// a block's scales are fetched once, not once per wave that uses them. Each
// run has its own record count (rows x 8 bytes) and a lane's whole offset
// (block row and lane) is range-checked against it, so rows past M or N
// fetch zeros, per lane; their results are never stored. alpha is 1.
//
// KW = 2: the two waves of a one-wave-tile block split every stage's K, wave
// k taking the 64-deep substeps of parity k, and the odd-substep partial
// sums reach the even-substep wave through LDS at the end (the even wave
// adds them and writes the tile). With one 32 x 32 tile of an M <= 32 call,
// this replaces a 64-row tile whose second wave only computed rows past M
// (same box, 6144 x 4096: M = 1 7.22 -> 7.15 us, M = 16 8.26 -> 8.15, M = 32
// 9.45 -> 9.38; 16 x 768 x 512 3.67 -> 3.62).
template <int BM, int BN, int WM, int WN, int NS, int GM, bool KTAIL, int NSUB, int AE = BM,
          bool GLU = false, bool ROPE = false, bool FP4 = false, bool WNT = false, int KW = 1>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * KW * 64) void gemm_kernel(GemmArgs a) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NQW = (BM / WM) * WAVES_N;  // waves with a tile of their own
  constexpr int NW = NQW * KW;
  static_assert(KW == 1 || (KW == 2 && NQW == 1 && !GLU && !FP4), "K split: one-wave tiles, split or RoPE form");
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int ROWS = AE + BN;  // LDS rows of a 128-deep sub-buffer: A, then B
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
  // the wave's tile (qw) and, with KW = 2, its substep parity (kslice)
  const int qw = wave % NQW, kslice = wave / NQW;
  const int wm0 = (qw / WAVES_N) * WM, wn0 = (qw % WAVES_N) * WN;

  // Epilogue operands. Read in the epilogue, they formed a chain behind the
  // last stage: the two scale loads, the split table one scalar load and
  // wait at a time, then the bias (RoPE: and the rope words of the lane's
  // rows). On small tiles (few waves, short K loops) that tail is visible,
  // so these kernels read them ahead of the main loop, where their latency
  // overlaps the weight stream. The loads are older than every ring load,
  // so the ring's vmcnt waits (in-order returns) stay exact.
  //  EARLY (FP8 split form, tiles of at most 64 x 64): alpha and each lane's
  //    bias bits here, its output column address and row stride (bytes)
  //    after the prologue's loads (same box: 6144 x 4096 at M = 1 7.53 ->
  //    7.19 us, M = 16 8.49 -> 8.25; 16 x 768 x 512 4.10 -> 3.67; 256 x 2560
  //    x 2048 bf16 9.27 -> 8.45; 256 x 2048 x 2048 7.36 -> 7.18; 256 x 2048
  //    x 8192 17.17 -> 16.96).
  //  EARLY_R (RoPE form, one 32 x 32 accumulator a wave: the 64 x 64 plan):
  //    alpha, the bias bits and the 16 (cos, sin) words (256 x 2560 x 2048
  //    + RoPE + cache: 9.83 -> 9.71 us).
  // The rest read them in the epilogue: 128 x 128 tiles (the registers held
  // across the loop cost more than the tail: 15.6 -> 16.0 us at 256 x 16384
  // x 2048), the one-row weight-streaming plan with all 64 A rows (M = 64:
  // 11.23 -> 11.31 us), the GEGLU form and the MXFP4 forms (no gain
  // measured; MXFP4 at M = 1 6.07 -> 6.18 us).
  constexpr bool SPLIT = !GLU && !ROPE;
  constexpr bool EARLY = SPLIT && !FP4 && BM * BN <= 64 * 64 && !(WNT && AE == 64);
  constexpr bool EARLY_R = ROPE && !FP4 && BM * BN <= 64 * 64 && MI * NJ == 1;
  constexpr int NE = EARLY ? NJ : 1;
  float alpha = 1.0f;
  uint16_t ep_b[NE], ep_rb = 0;
  uint32_t ep_cs[EARLY_R ? 16 : 1];
  gbyte_t* ep_col[NE];
  int64_t ep_ld[NE];
  // the scales and the raw bias bits, loaded with no branch (from the
  // weights when there is no bias: any readable address; the epilogue then
  // ignores them) and converted only in the epilogue, so nothing waits for
  // them early
  auto ep_loads = [&]() {
    alpha = FP4 ? 1.0f : (*a.act_scale) * (*a.w_scale);
    if constexpr (EARLY) {
      const uint16_t* bsrc = a.bias != nullptr ? a.bias : reinterpret_cast<const uint16_t*>(a.w);
#pragma unroll
      for (int j = 0; j < NJ; ++j) ep_b[j] = bsrc[min(n0 + wn0 + j * 32 + (lane & 31), a.N - 1)];
    }
    if constexpr (EARLY_R) {
      // every lane reads its rope words (v columns too, whose values the
      // epilogue ignores): rows clamped to M - 1, columns to an even d < hd
      const uint16_t* bsrc = a.bias != nullptr ? a.bias : reinterpret_cast<const uint16_t*>(a.w);
      const int n = n0 + wn0 + (lane & 31);
      ep_rb = bsrc[min(n, a.N - 1)];
      const uint16_t* rp = a.rope + ((n % a.hd) & ~1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = min(m0 + wm0 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3), a.M - 1);
        ep_cs[r] = *reinterpret_cast<const uint32_t*>(rp + (int64_t)m * a.hd);
      }
    }
  };
  // split form: the split owning each of this lane's columns, by a
  // run-time loop over the call's splits (one scalar load of each entry,
  // selects per lane: a fully unrolled scan over the whole table held it
  // in scalar registers and spilled them)
  auto ep_splits = [&]() {
    if constexpr (EARLY) {
      const int esz = a.out_f32 ? 4 : 2;
      int nv[NE];
      uint64_t bv[NE];
      int64_t lv[NE];
      int ov[NE];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        nv[j] = n0 + wn0 + j * 32 + (lane & 31);
        bv[j] = reinterpret_cast<uint64_t>(a.sp.ptr[0]);
        lv[j] = a.sp.ld[0];
        ov[j] = 0;
      }
#pragma unroll 1
      for (int s = 1; s < a.sp.n; ++s) {
        const int so = a.sp.off[s];
        const uint64_t sp = reinterpret_cast<uint64_t>(a.sp.ptr[s]);
        const int64_t sl = a.sp.ld[s];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bool t = nv[j] >= so;
          bv[j] = t ? sp : bv[j];
          lv[j] = t ? sl : lv[j];
          ov[j] = t ? so : ov[j];
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        ep_col[j] = reinterpret_cast<gbyte_t*>(bv[j] + (uint64_t)((int64_t)(nv[j] - ov[j]) * esz));
        ep_ld[j] = lv[j] * esz;
      }
    }
  };
  if constexpr (EARLY || EARLY_R) ep_loads();

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
        const int u = wave + (A ? j : j - LPA) * NW + (A ? 0 : AE / 8);
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
        // WNT (plans with one row of tiles, where each weight byte is read
        // by one block): weight loads carry the non-temporal hint, so the
        // stream allocates nothing in the caches (6144 x 4096 weights,
        // rotated: M = 1 8.5 -> 7.9 us, M = 16 9.3 -> 8.5, M = 64 12.5 ->
        // 11.6); with several rows of tiles sharing a weight tile through
        // L2 it costs (256 x 2560 x 2048: 8.5 -> 10.7 us)
        if (A)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, WNT ? 2 : 0);
      }
      if constexpr (FP4) {
        // the scales of run kt * NSUB + q: 32 rows (256 bytes) per load
        const int64_t run = kt * NSUB + q;
        uint8_t* sdst = smem + SCBASE + (SL * NSUB + q) * SCB;
#pragma unroll
        for (int k = 0; k < SCL; ++k) {
          const __amdgpu_buffer_rsrc_t r = make_rsrc(sc_src[k] + run * sc_run[k], sc_rec[k]);
          // the block's row offset rides in the lane offset, which the raw
          // buffer range check covers (the scalar offset is not checked):
          // rows past M or N fetch zeros and nothing past the run is read
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(sdst + sc_lds[k]), 4, sc_lane + sc_off[k], 0, 0, 0);
        }
      }
    }
  };
  // operand read of substep SUB from slot SL: two 16-byte chunks per lane
  const int lrow32 = lane & 31;
  const int sw = (lrow32 >> 1) & 7;  // (row >> 1) & 7 for rows 32k + lrow32
  const uint8_t* lbase0 = smem + lrow32 * 128 + ((((lane >> 5) * 2) ^ sw) * 16);
  const uint8_t* lbase1 = smem + lrow32 * 128 + ((((lane >> 5) * 2 + 4) ^ sw) * 16);
  const uint8_t* lbk = kslice ? lbase1 : lbase0;  // KW = 2: this wave's half of each 128-deep run
  // this lane's scale dword within a 32-row block: row lrow32, K half l / 32
  const uint8_t* sbase = smem + SCBASE + lane * 4;
  // first LDS row of A fragment i of this wave (row 0 past the loaded rows)
  auto arow = [&](int i) { return (AE == BM || wm0 + i * 32 < AE) ? wm0 + i * 32 : 0; };
  auto read_frags = [&](auto SLC, auto SUBC, auto* af, auto* bf) {
    constexpr int SL = decltype(SLC)::value, SUB = decltype(SUBC)::value;
    if constexpr (FP4) {
      // step SUB % 4 of sub-buffer SUB / 4: chunk 2 (SUB % 4) + l / 32
      const uint8_t* lb = smem + lrow32 * 128 + ((((SUB & 3) * 2 + (lane >> 5)) ^ sw) * 16) + SL * STAGE +
                          (SUB >> 2) * SUBB;
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *reinterpret_cast<const v4i*>(lb + (AE + wn0 + j * 32) * 128);
#pragma unroll
      for (int i = 0; i < MI; ++i) af[i] = *reinterpret_cast<const v4i*>(lb + arow(i) * 128);
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
    // KW = 2: SUB counts this wave's substeps (global substep 2 SUB + kslice)
    const uint8_t* lb = (KW == 2 ? lbk : ((SUB & 1) ? lbase1 : lbase0)) + SL * STAGE +
                        (KW == 2 ? SUB : (SUB >> 1)) * SUBB;
    // the second chunk sits at position ^ 1, i.e. +16 or -16 bytes
    const int d1 = (sw & 1) ? -16 : 16;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint8_t* rowp = lb + (AE + wn0 + j * 32) * 128;
      const v4i lo = *reinterpret_cast<const v4i*>(rowp);
      const v4i hi = *reinterpret_cast<const v4i*>(rowp + d1);
      bf[j] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const uint8_t* rowp = lb + arow(i) * 128;
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
  constexpr int KSUB = (FP4 ? 4 : 2) * NSUB / KW;  // 64-deep substeps a wave multiplies per stage
  constexpr bool ALL = MI * NJ * KSUB <= 8;
  static_assert(KW == 1 || ALL, "K split: fragments of the whole stage read at once");
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
  if constexpr (EARLY) ep_splits();
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
  if constexpr (KW == 2) {
    // the odd-substep wave's sums go through the ring slot that no load
    // targets and no wave reads any more (that of stage KT, as the epilogue
    // uses it); the even wave adds them to its own (a fixed order)
    float* red = reinterpret_cast<float*>(smem + (KT % NS) * STAGE);
    static_assert(MI * NJ * 16 * 64 * 4 <= STAGE, "partial sums fit one slot");
    if (kslice == 1) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((i * NJ + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (kslice == 1) return;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += red[((i * NJ + j) * 16 + r) * 64 + lane];
  }

  if constexpr (!EARLY && !EARLY_R) ep_loads();
  {
    constexpr int SLOT = STAGE, TOTAL = NS * STAGE;
    uint8_t* slot = smem + (KT % NS) * STAGE;
    uint8_t* lds = smem;
#include "frt_gemm_epilogue.inc"
  }
}

// The split table in LDS: the 256 x 256 kernel's epilogue looks a column's
// split up there (lane by lane) instead of keeping the table's 80 scalar
// registers live next to 256 accumulator registers.
struct LdsSplits {
  uint64_t ptr[FRT_MAX_SPLITS];
  int64_t ld[FRT_MAX_SPLITS];
  int off[FRT_MAX_SPLITS];
  int n;
  uint8_t grp[32];  // the split of each 8-column group of a (<= 256-column) tile
};

// Output pointer of column n (in its split) and its row stride, in bytes
// of `esize`-byte elements.
__device__ __forceinline__ void split_of(const LdsSplits* t, int n, int esize, uint8_t*& colp, int64_t& ldb) {
  const int ns = t->n;
  int idx = 0;
#pragma unroll
  for (int s = 1; s < FRT_MAX_SPLITS; ++s)
    if (s < ns && n >= t->off[s]) idx = s;
  colp = reinterpret_cast<uint8_t*>(t->ptr[idx]) + (int64_t)(n - t->off[idx]) * esize;
  ldb = t->ld[idx] * esize;
}

// Two floats as packed bf16, low half first, by the conversion instruction
// (v_cvt_pk_bf16_f32): round to nearest even, the same bits as f2bf for
// every non-NaN input (checked over all 2^32 patterns on the device); a
// NaN stays a NaN but keeps its payload bits where f2bf returns 0x7fc0.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Epilogue of the 256 x 256 kernel: out = alpha * acc + bias in the split,
// GEGLU or RoPE form (the forms described at gemm_kernel). The kernel's
// MFMAs take the B fragment as their first operand, so lane l holds output
// row 16i + l % 16 of accumulator (i, j) and four consecutive columns of
// it: for the GEGLU form columns 16j + 4q + r (q = l / 16, r = 0..3); for
// the split and RoPE forms the B tile's rows are loaded in an order (see
// the kernel) that gives accumulators 2p and 2p + 1 the columns 32p + 8q +
// r and 32p + 8q + 4 + r, eight consecutive columns a lane. Each lane
// writes its values straight to memory with no staging. Split form: with
// vec_out (bf16, split widths, offsets and strides multiples of 8) 16 bytes
// a store, else one store per element; `tab` is the split table in LDS,
// filled here after a block barrier. Rows past M exist only in the last row
// of tiles.
template <bool GLU, bool ROPE, int NJ, int BN>
__device__ __forceinline__ void gemm256_epilogue(const GemmArgs& a, v4f (&acc)[8][NJ], int m0, int n0, int wm0,
                                                 int wn0, int lane, LdsSplits* tab) {
  constexpr int MI = 8;
  const int c4 = (lane >> 4) * 4;            // GEGLU: first of the lane's columns in a fragment
  const int c8 = (lane >> 4) * 8;            // split, RoPE: first of its columns in a fragment pair
  const int mr = m0 + wm0 + (lane & 15);     // the lane's row in row block i = 0
  const bool rows_in = m0 + wm0 + 128 <= a.M;
  const float alpha = (*a.act_scale) * (*a.w_scale);
  // split / RoPE column of value r of accumulator column block j
  auto col = [&](int j, int r) { return n0 + wn0 + (j >> 1) * 32 + c8 + (j & 1) * 4 + r; };
  if constexpr (ROPE) {
    const int nq = a.nh * a.hd, nk = a.kv * a.hd;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // the rotary pair (n, n + 1): n even, both in one of q, k, v
        const int n = col(j, 2 * t);
        if (n >= a.N) continue;
        const bool rot = n < nq + nk;
        const int d = n % a.hd;
        const float be = a.bias != nullptr ? bf16f(a.bias[n]) : 0.0f;
        const float bo = a.bias != nullptr ? bf16f(a.bias[n + 1]) : 0.0f;
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
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int m = mr + i * 16;
          if (!rows_in && m >= a.M) continue;
          const float ve = __uint_as_float(f2bf(alpha * acc[i][j][2 * t] + be) << 16);
          const float vo = __uint_as_float(f2bf(alpha * acc[i][j][2 * t + 1] + bo) << 16);
          float oe = ve, oo = vo;
          if (rot) {
            // a' = a c - b s on the even column, b' = b c + a s on the odd one
            const uint32_t cs = *reinterpret_cast<const uint32_t*>(a.rope + (int64_t)m * a.hd + d);
            oe = __builtin_fmaf(ve, bf16lo(cs), -1.0f * (vo * bf16hi(cs)));
            oo = __builtin_fmaf(vo, bf16lo(cs), 1.0f * (ve * bf16hi(cs)));
          }
          dst[(int64_t)m * ld] = (uint16_t)f2bf(oe);
          dst[(int64_t)m * ld + 1] = (uint16_t)f2bf(oo);
        }
      }
    }
    return;
  }
  if constexpr (GLU) {
    // gate and up rounded to bf16 as the unfused GEMM output would be, then
    // the GEGLU quantiser of frt_ffn.hip; accumulators 2p (gate) and 2p + 1
    // (up) hold the same four gate columns
    const float qs = *a.q_scale, qr = 1.0f / qs;
    const bool vec4 = ((reinterpret_cast<uintptr_t>(a.q8) | (uintptr_t)a.ld_q8) & 3) == 0;
    // the biases first (the compiler cannot move their loads above the
    // code stores)
    float bg[NJ / 2][4], bu[NJ / 2][4];
#pragma unroll
    for (int p = 0; p < NJ / 2; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gc = n0 + (wn0 >> 1) + p * 16 + c4 + r;
        const bool ok = a.bias != nullptr && gc < a.H;
        bg[p][r] = ok ? bf16f(a.bias[gc]) : 0.0f;
        bu[p][r] = ok ? bf16f(a.bias[a.H + gc]) : 0.0f;
      }
    // the wave's 64 gate columns and 128 rows all in range, 4-byte code
    // stores: no per-value checks (a uniform branch)
    const bool all_in = rows_in && vec4 && n0 + (wn0 >> 1) + 64 <= a.H;
    auto body = [&](auto ALLC) {
      constexpr bool ALL = decltype(ALLC)::value;
#pragma unroll
      for (int p = 0; p < NJ / 2; ++p) {
        const int gc = n0 + (wn0 >> 1) + p * 16 + c4;
        if (!ALL && gc >= a.H) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int m = mr + i * 16;
          if (!ALL && m >= a.M) continue;
          float qv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // gate and up to bf16 in one conversion (pk_bf16 rounds as f2bf)
            const uint32_t w = pk_bf16(alpha * acc[i][2 * p][r] + bg[p][r], alpha * acc[i][2 * p + 1][r] + bu[p][r]);
            const float y = gelu_tanh(bf16lo(w)) * bf16hi(w);
            qv[r] = clamp_fp8(div_rn(y, qs, qr));
          }
          const uint32_t codes = cvt4_fp8(qv[0], qv[1], qv[2], qv[3]);
          uint8_t* q = a.q8 + (int64_t)m * a.ld_q8 + gc;
          if (ALL || (vec4 && gc + 4 <= a.H)) {
            *reinterpret_cast<uint32_t*>(q) = codes;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (gc + r < a.H) q[r] = (uint8_t)(codes >> (8 * r));
          }
        }
      }
    };
    if (all_in)
      body(std::true_type{});
    else
      body(std::false_type{});
    return;
  }
  if (threadIdx.x < FRT_MAX_SPLITS) {
    tab->ptr[threadIdx.x] = reinterpret_cast<uint64_t>(a.sp.ptr[threadIdx.x]);
    tab->ld[threadIdx.x] = a.sp.ld[threadIdx.x];
    tab->off[threadIdx.x] = a.sp.off[threadIdx.x];
    if (threadIdx.x == 0) tab->n = a.sp.n;
  } else if (threadIdx.x >= 64 && threadIdx.x < 64 + BN / 8 && a.vec_out) {
    // vec_out split widths are multiples of 8: an 8-column group lies in one
    // split, found once here for the whole block
    const int g = threadIdx.x - 64, n = n0 + 8 * g;
    int idx = 0;
#pragma unroll
    for (int sp = 1; sp < FRT_MAX_SPLITS; ++sp)
      if (sp < a.sp.n && n >= a.sp.off[sp]) idx = sp;
    tab->grp[g] = (uint8_t)idx;
  }
  __syncthreads();
  if (a.vec_out) {
    // every 8-column chunk's split and bias first (the compiler cannot move
    // these loads above the output stores, which might alias them)
    constexpr int NP = NJ / 2;
    uint8_t* colp[NP];
    int64_t ldb[NP];
    float b[NP][8];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // columns n .. n + 7: one 8-column group, in one split
      const int n = col(2 * p, 0);
      const int idx = tab->grp[(n - n0) >> 3];
      ldb[p] = tab->ld[idx] * 2;
      colp[p] = reinterpret_cast<uint8_t*>(tab->ptr[idx]) + (int64_t)(n - tab->off[idx]) * 2 + (int64_t)mr * ldb[p];
    }
    if (a.bias != nullptr) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int n = col(2 * p, 0), nb = n < a.N ? n : 0;  // N >= 8
#pragma unroll
        for (int r = 0; r < 8; ++r) b[p][r] = bf16f(a.bias[nb + r]);
      }
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int r = 0; r < 8; ++r) b[p][r] = 0.0f;
    }
    // rows checked only in the last row of tiles (a uniform branch)
    auto store_vec = [&](auto ALLC) {
      constexpr bool ALL = decltype(ALLC)::value;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (col(2 * p, 0) >= a.N) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (!ALL && mr + i * 16 >= a.M) continue;
          const v4f& lo = acc[i][2 * p];
          const v4f& hi = acc[i][2 * p + 1];
          const u32x4_t v = {pk_bf16(alpha * lo[0] + b[p][0], alpha * lo[1] + b[p][1]),
                             pk_bf16(alpha * lo[2] + b[p][2], alpha * lo[3] + b[p][3]),
                             pk_bf16(alpha * hi[0] + b[p][4], alpha * hi[1] + b[p][5]),
                             pk_bf16(alpha * hi[2] + b[p][6], alpha * hi[3] + b[p][7])};
          // a global (not flat) store: the split table holds generic
          // pointers. Non-temporal: the step's outputs are not read again
          // by this launch, and streaming them past the caches keeps the
          // end-of-round store bursts off the operand traffic (cold outputs,
          // 8192 x 9216 x 3072 + bias: 205.8 -> 192.6 us; 2048 x 9216 x
          // 4096: 83.7 -> 78.6 us)
          __builtin_nontemporal_store(
              v, (__attribute__((address_space(1))) u32x4_t*)(uintptr_t)(colp[p] + (int64_t)(i * 16) * ldb[p]));
        }
      }
    };
    if (rows_in)
      store_vec(std::true_type{});
    else
      store_vec(std::false_type{});
    return;
  }
  // one store per element (fp32 output, or splits not on 8-column bounds)
  auto store_all = [&](auto F32C) {
    constexpr bool F32 = decltype(F32C)::value;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = col(j, r);
        if (n >= a.N) continue;
        uint8_t* colp;
        int64_t ldb;
        split_of(tab, n, F32 ? 4 : 2, colp, ldb);
        const float b = a.bias != nullptr ? bf16f(a.bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int m = mr + i * 16;
          if (!rows_in && m >= a.M) continue;
          const float v = alpha * acc[i][j][r] + b;
          if constexpr (F32)
            *reinterpret_cast<float*>(colp + (int64_t)m * ldb) = v;
          else
            *reinterpret_cast<uint16_t*>(colp + (int64_t)m * ldb) = (uint16_t)f2bf(v);
        }
      }
  };
  if (a.out_f32)
    store_all(std::true_type{});
  else
    store_all(std::false_type{});
}

// Large-M FP8 kernel: a 256 x BN block tile (BN = 256, 192 or 128) of four
// 128 x BN/2 wave tiles (one wave per SIMD, accumulators in the
// matrix-core registers), on v_mfma_f32_16x16x128_f8f6f4: each MFMA takes a
// whole 128-deep stage of a 16-row A fragment and a 16-row B fragment.
// Under sustained load the board holds an FP8 MFMA loop of this shape at a
// higher engine clock than one of 32x32x64 MFMAs doing the same work
// (measured: 2.05 against 1.86 GHz), and this kernel's time follows the
// clock.
//
// The LDS is a ring of five 32 KB units; a unit holds the A rows (256) or
// the B rows (BN) of one 128-deep stage, 128 bytes a row in the swizzled
// row layout of gemm_kernel. Unit u sits in slot u % 5; stage kt reads
// units 2kt (A) and 2kt + 1 (B). During stage kt the wave issues the loads
// of units 2kt + 4 and 2kt + 5 (the next-but-one stage), so a unit is in
// flight for 1.5-1.75 stages before its first read.
//
// A wave's tile is four blocks over quarters of its fragments (A lo / A hi:
// fragment rows 0-63 / 64-127; B lo / B hi: the first and second half of
// its BN/2 rows), in the order (A lo, B lo), (A hi, B lo), (A lo, B hi),
// (A hi, B hi), four register quarters (at most 128 VGPRs) in all. Block 0
// issues the loads of unit 2kt + 4 (its slot, unit 2kt - 1's, freed at the
// previous stage's first barrier) and reads the stage's A hi and B hi, which
// ends the reads of units 2kt and 2kt + 1; a barrier frees their slots;
// block 1 issues unit 2kt + 5 into unit 2kt's slot; after block 2 the wave
// waits for units up to 2kt + 3 and takes a second barrier; block 3, which
// needs neither, reads the next stage's A lo and B lo. Work is issued in a
// fixed order (no compiler reordering). Each accumulator takes one MFMA per
// stage, in K order. Past the last stage the loads fetch zeros into free
// slots (branch-free); the block drains them before the epilogue.
//
// GLU and ROPE select the epilogue forms described at gemm_kernel (BN = 256
// only); for GLU the B tile interleaves 16 gate rows and the 16 matching up
// rows, so each lane holds a gate column and its up column. KTAIL
// zero-fills the 16-byte chunks past K.
template <bool GLU, bool ROPE, bool KTAIL, int BN = 256>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm256_kernel(GemmArgs a) {
  static_assert(BN == 256 || ((BN == 192 || BN == 128) && !GLU && !ROPE), "narrower tiles: split form only");
  constexpr int BM = 256, GM = 4, NW = 4, MI = 8, WN = BN / 2, NJ = WN / 16, NQ = NJ / 2;
  constexpr int UNIT = 256 * 128, RU = 5;
  constexpr int LPA = BM / 8 / NW, LPB = BN / 8 / NW;  // loads a wave per A / B unit
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RU * UNIT];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N - a.n_base + BN - 1) / BN;
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * WN;
  const uint32_t x_bytes = (uint32_t)((int64_t)(a.M - 1) * a.ld_x + a.K);
  const uint32_t w_bytes = (uint32_t)((int64_t)a.N * a.K);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, w_bytes);
  // load j of a unit covers tile rows 8g .. 8g + 7, g = wave + 4j; with g's
  // parity that of the wave, (row >> 1) & 7 = ((wave & 1) << 2) | (lrow >> 1)
  const int lrow = lane >> 3;
  const int cch = (lane & 7) ^ (((wave & 1) << 2) | (lrow >> 1));
  const uint32_t stepA = (uint32_t)(8 * NW) * (uint32_t)a.ld_x;
  const uint32_t stepB = (uint32_t)(8 * NW) * (uint32_t)a.K;
  const int KT = (a.K + 127) / 128;
  // One tile per block: a block that ends leaves its stores draining while
  // the CU's next block loads (a loop over tiles inside one block would
  // have to wait for them: loads and stores share the wait counter).
  // m0, n0: the tile's first output row and column (GLU: first gate column)
  const TileXY t = tile_of(blockIdx.x, tiles_m, tiles_n, GM);
  const int m0 = t.tm * BM, n0 = a.n_base + t.tn * (GLU ? BN / 2 : BN);
  const uint32_t offA = (uint32_t)((int64_t)(m0 + wave * 8 + lrow) * a.ld_x) + cch * 16;
  // B rows: GLU forms map each load's rows in ld below; the split and RoPE
  // forms put W row 32j + 16 (wave % 2) + 8 (lrow / 4) + 4 (wave / 2) +
  // lrow % 4 into tile row 32j + 8 wave + lrow (load j), so that fragment
  // rows 4q..4q+3 of fragments 2p and 2p + 1 are columns 32p + 8q .. + 7
  // (a wave's B rows start on a 32-row boundary)
  const uint32_t offB =
      GLU ? (uint32_t)(lrow * a.K + cch * 16)
          : (uint32_t)((int64_t)(n0 + 16 * (wave & 1) + 8 * (lrow >> 2) + 4 * (wave >> 1) + (lrow & 3)) * a.K) +
                cch * 16;
  // this lane's offset for load 0 of the A (B = false) or B unit of stage
  // ks, or kOOB past the last stage (and, with KTAIL, past K). Load j adds
  // a multiple of the row stride that leaves kOOB past any record count
  // (the host bounds M (M >= 512 here), K and ld_x: under 2^31 - 224 row
  // strides), so a unit's zero fill needs one select, not one per load.
  auto ubase = [&](auto BC, int ks) {
    constexpr bool B = decltype(BC)::value;
    const int k0 = ks * 128;
    uint32_t o = (B ? offB : offA) + k0;
    if constexpr (KTAIL) {
      if (k0 + cch * 16 >= a.K) o = kOOB;
    }
    return ks < KT ? o : kOOB;
  };
  // load j of a unit whose ubase is `ob` into the ring slot at byte offset
  // `so`
  auto ld = [&](int so, auto BC, uint32_t ob, int j) {
    constexpr bool B = decltype(BC)::value;
    uint8_t* dst = smem + so + (wave + j * NW) * 1024;
    uint32_t o;
    if constexpr (B) {
      if constexpr (GLU) {
        // B unit g: 16-column group g / 4, gate or up half by (g / 2) % 2,
        // 8-row group g % 2
        const int g = wave + j * NW;
        const int row = ((g >> 1) & 1) * a.H + n0 + (g >> 2) * 16 + (g & 1) * 8;
        o = ob + (uint32_t)row * (uint32_t)a.K;
      } else {
        o = ob + j * stepB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
    } else {
      o = ob + j * stepA;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)dst, 16, o, 0, 0, 0);
    }
  };
  // fragment lanes: row lane % 16 of a 16-row fragment, 32-byte K group
  // lane / 16 (chunks 2g and 2g + 1 of the 128-byte row); the row's swizzle
  // key (row >> 1) & 7 is (lane % 16) / 2 for every fragment
  const int r16 = lane & 15, sw = r16 >> 1;
  const int lo = r16 * 128 + ((((lane >> 4) * 2) ^ sw) * 16);
  // the fragment's second chunk sits at position ^ 1, i.e. +16 or -16 bytes
  const int d1 = (sw & 1) ? -16 : 16;
  v8i R[4][4];  // four quarters of (up to) four fragments
  v4f acc[MI][NJ];
  // 16-byte half h of quarter Q: fragment h / 2 of the rows from row0 of
  // `unit` (which includes this lane's offset), part h % 2
  auto rd = [&](auto QC, const uint8_t* unit, int row0, int h) {
    constexpr int Q = decltype(QC)::value;
    const int k = h >> 1;
    const v4i v = *reinterpret_cast<const v4i*>(unit + (row0 + k * 16) * 128 + ((h & 1) ? d1 : 0));
    if (h & 1)
      R[Q][k].hi = v;
    else
      R[Q][k].lo = v;
  };
  // MFMA of accumulator (i0 + i, j0 + j) on fragment i of quarter QA and
  // fragment j of quarter QB, the B fragment first (so that a lane's
  // results run along an output row)
  auto mf = [&](auto QAC, auto QBC, int i0, int j0, int i, int j) {
    constexpr int QA = decltype(QAC)::value, QB = decltype(QBC)::value;
    acc[i0 + i][j0 + j] =
        __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(R[QB][j], R[QA][i], acc[i0 + i][j0 + j], 0, 0, 0, 0, 0, 0);
  };
  // MFMA order within a block (4 x NQ): shells k = 0..3 ((k, 0..k) then
  // (0..k-1, k), columns < NQ), so the first MFMAs need the fragments read
  // first
  constexpr int NB = 4 * NQ;  // MFMAs a block
  constexpr int OI4[16] = {0, 1, 1, 0, 2, 2, 2, 0, 1, 3, 3, 3, 3, 0, 1, 2};
  constexpr int OJ4[16] = {0, 0, 1, 1, 0, 1, 2, 2, 2, 0, 1, 2, 3, 3, 3, 3};
  constexpr int OI3[12] = {0, 1, 1, 0, 2, 2, 2, 0, 1, 3, 3, 3};
  constexpr int OJ3[12] = {0, 0, 1, 1, 0, 1, 2, 2, 2, 0, 1, 2};
  constexpr int OI2[8] = {0, 1, 1, 0, 2, 2, 3, 3};
  constexpr int OJ2[8] = {0, 0, 1, 1, 0, 1, 0, 1};
  auto oi = [&](int q) { return NQ == 4 ? OI4[q] : NQ == 3 ? OI3[q] : OI2[q]; };
  auto oj = [&](int q) { return NQ == 4 ? OJ4[q] : NQ == 3 ? OJ3[q] : OJ2[q]; };
  // the next stage's A lo / B lo half-reads in the order A0 B0 A1 B1 ...
  // (B only for fragments < NQ): read n (0 .. 8 + 2 NQ - 1) is half h of
  // quarter 0 (A) or 1 (B)
  auto lo_read = [&](int n, const uint8_t* una, const uint8_t* unb) {
    const int pair = n >> 1, part = n & 1;
    // pairs alternate A, B while both remain, then A only
    const int ab = pair < 2 * NQ ? (pair & 1) : 0;
    const int k = pair < 2 * NQ ? (pair >> 1) : pair - NQ;
    if (ab == 0)
      rd(std::integral_constant<int, 0>{}, una, wm0, 2 * k + part);
    else
      rd(std::integral_constant<int, 1>{}, unb, wn0, 2 * k + part);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using BA = std::false_type;
  using BB = std::true_type;
  // unit u sits in ring slot u % RU; slot offsets in bytes, advanced by
  // one unit with a wrap (no division in the loop)
  auto nx = [](int so) { return so + UNIT == RU * UNIT ? 0 : so + UNIT; };
  // stage kt, whose A unit 2kt sits at slot offset sa: quarter 0 holds A
  // lo, 1 B lo, 2 A hi, 3 B hi
  auto stage = [&](int kt, int sa) {
    const int sb = nx(sa), sna = nx(sb), snb = nx(sna), s4 = nx(snb);
    const uint8_t* ua = smem + sa + lo;
    const uint8_t* ub = smem + sb + lo;
    const uint8_t* una = smem + sna + lo;
    const uint8_t* unb = smem + snb + lo;
    const uint32_t oa2 = ubase(BA{}, kt + 2), ob2 = ubase(BB{}, kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    // (A lo, B lo); the loads of unit 2kt + 4 (its slot, unit 2kt - 1's,
    // was freed at the previous stage's first barrier); this stage's A hi
    // and B hi, which finish the reads of units 2kt and 2kt + 1
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      mf(I0{}, I1{}, 0, 0, oi(q), oj(q));
      if ((q & 1) == 0 && (q >> 1) < LPA) ld(s4, BA{}, oa2, q >> 1);
      if (q < 8)
        rd(I2{}, ua, wm0 + 64, q);
      else
        rd(I3{}, ub, wn0 + NQ * 16, q - 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = NB / 2; j < LPA; ++j) ld(s4, BA{}, oa2, j);
#pragma unroll
    for (int h = NB - 8; h < 2 * NQ; ++h) rd(I3{}, ub, wn0 + NQ * 16, h);
    // every wave done with units 2kt and 2kt + 1
    __builtin_amdgcn_s_waitcnt(lgkm_imm(0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // (A hi, B lo) with the loads of unit 2kt + 5 (into unit 2kt's slot),
    // then (A lo, B hi)
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      mf(I2{}, I1{}, 4, 0, oi(q), oj(q));
      if ((q & 1) == 0 && (q >> 1) < LPB) ld(sa, BB{}, ob2, q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = NB / 2; j < LPB; ++j) ld(sa, BB{}, ob2, j);
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      mf(I0{}, I3{}, 0, NQ, oi(q), oj(q));
      __builtin_amdgcn_sched_barrier(0);
    }
    // units up to 2kt + 3 landed (this wave's last LPA + LPB loads are
    // units 2kt + 4 and 2kt + 5)
    __builtin_amdgcn_s_waitcnt(vm_imm(LPA + LPB));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // (A hi, B hi); the next stage's A lo and B lo into their quarters
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      mf(I2{}, I3{}, 4, NQ, oi(q), oj(q));
      lo_read(q, una, unb);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int n = NB; n < 8 + 2 * NQ; ++n) lo_read(n, una, unb);
  };

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
  // prologue: units 0..3 in flight; once units 0 and 1 landed, stage 0's
  // A lo and B lo
#pragma unroll
  for (int j = 0; j < LPA; ++j) ld(0, BA{}, ubase(BA{}, 0), j);
#pragma unroll
  for (int j = 0; j < LPB; ++j) ld(UNIT, BB{}, ubase(BB{}, 0), j);
#pragma unroll
  for (int j = 0; j < LPA; ++j) ld(2 * UNIT, BA{}, ubase(BA{}, 1), j);
#pragma unroll
  for (int j = 0; j < LPB; ++j) ld(3 * UNIT, BB{}, ubase(BB{}, 1), j);
  __builtin_amdgcn_s_waitcnt(vm_imm(LPA + LPB));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int n = 0; n < 8 + 2 * NQ; ++n) lo_read(n, smem + lo, smem + UNIT + lo);
  for (int kt = 0, sa = 0; kt < KT; ++kt, sa = nx(nx(sa))) stage(kt, sa);
  // drain the zero-fill loads past the last stage; then every wave is done
  // with the ring and the epilogue may stage in any of it
  __builtin_amdgcn_s_waitcnt(vm_imm(0));
  __syncthreads();
  gemm256_epilogue<GLU, ROPE, NJ, BN>(a, acc, m0, n0, wm0, wn0, lane, reinterpret_cast<LdsSplits*>(smem));
}

// The 256 x 256 plan runs on gemm256_kernel at every K the API admits: it
// beat a 256 x 256 tile of eight 128 x 64 waves (32x32x64 MFMAs, the same
// direct-store improvements to its epilogue) down to K = 512 (rotated
// operands, same box: 8192 x 9216 x 512 / 1024: 72.6 -> 67.6, 102.0 -> 94.0
// us; 2048 x 32768 x 512 / 1024: 62.2 -> 55.8, 87.0 -> 78.0 us).
template <bool GLU, bool ROPE, int BN = 256>
hipError_t launch_256(const GemmArgs& a, hipStream_t st) {
  const int tiles = ((a.M + 255) / 256) * ((a.N - a.n_base + BN - 1) / BN);
  if (a.K % 128 == 0)
    hipLaunchKernelGGL((gemm256_kernel<GLU, ROPE, false, BN>), dim3(tiles), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm256_kernel<GLU, ROPE, true, BN>), dim3(tiles), dim3(256), 0, st, a);
  return hipGetLastError();
}

// Rounds of 256 x BN tiles on `cus` CUs.
int64_t rounds_256(const GemmArgs& a, int BN, int cus) {
  const int64_t tiles = (int64_t)((a.M + 255) / 256) * ((a.N + BN - 1) / BN);
  return (tiles + cus - 1) / cus;
}
template <int BM, int BN, int WM, int WN, int NS, int GM, int NSUB = 1, int AE = BM, bool GLU = false,
          bool ROPE = false, bool FP4 = false, bool WNT = false, int KW = 1>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t st) {
  // (GLU: N = 2H, so this is also ceil(H / (BN / 2)) column tiles)
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int threads = (BM / WM) * (BN / WN) * KW * 64;
  if constexpr (FP4) {  // whole stages (K a multiple of 256 * NSUB) is checked by the caller
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, GM, false, NSUB, AE, GLU, ROPE, true, WNT, KW>), dim3(tiles),
                       dim3(threads), 0, st, a);
    return hipGetLastError();
  }
  if (a.K % (128 * NSUB) == 0)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, GM, false, NSUB, AE, GLU, ROPE, false, WNT, KW>), dim3(tiles),
                       dim3(threads), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, GM, true, NSUB, AE, GLU, ROPE, false, WNT, KW>), dim3(tiles),
                       dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// The current plans use no workspace (the argument is kept in the ABI).
size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

// Compute units of the current device, cached per device. Threads that race
// on a device's first query each store the same count; the relaxed atomic
// makes those concurrent stores and loads well defined.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    c = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
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
//  M > 64: the plan of least per-CU load (plan_cost) among 256x256 tiles
//    (M >= 512 only: the MFMA-bound shapes; gemm256_kernel's four 128x128
//    waves), 128x128 of
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
      case 0:
        // split form: 256 x 192 tiles where they fill the same number of
        // rounds (at least two) better (same box: 8192 x 3072 x 3072 77.0 ->
        // 71.5 us, 2048 x 9216 x 4096 89.8 -> 77.3, 4096 x 6144 x 1024 39.3
        // -> 37.3); with more rounds (8192 x 9216 x 3072: 5 against 6) or a
        // single one (2000 x 5000 x 2048: 57.1 against 69.7 us) 256 x 256
        if constexpr (!ROPE) {
          const int64_t r256 = rounds_256(a, 256, cus);
          if (r256 >= 2 && rounds_256(a, 192, cus) == r256) return launch_256<false, false, 192>(a, st);
          // else, with a partial last round, two launches: 256 x 256 tiles
          // over the first columns, in whole rounds, then one round of
          // 256 x 128 tiles over the rest (8192 x 9216 x 3072: 1024 + 256
          // tiles instead of 1152 in 4.5 rounds)
          const int tm = (a.M + 255) / 256, tn = (a.N + 255) / 256;
          if (r256 >= 2 && ((int64_t)tm * tn) % cus != 0) {
            int nm = tn - 1;
            while (nm > 0 && ((int64_t)tm * nm) % cus != 0) --nm;
            const int64_t rest = (int64_t)tm * ((a.N - nm * 256 + 127) / 128);
            if (nm > 0 && rest <= cus && ((int64_t)tm * nm) / cus + 1 <= r256) {
              GemmArgs head = a;
              head.N = nm * 256;
              hipError_t e = launch_256<false, false, 256>(head, st);
              if (e != hipSuccess) return e;
              GemmArgs tail = a;
              tail.n_base = nm * 256;
              return launch_256<false, false, 128>(tail, st);
            }
          }
        }
        return launch_256<false, ROPE>(a, st);
      case 1: return launch_tiles<128, 128, 32, 32, 3, 2, 1, 128, false, ROPE>(a, st);
      // tile rows rastered in pairs (GM = 2): an XCD's run of tiles covers
      // two tile rows of each weight column it touches, so a weight tile
      // reaches fewer XCD caches than with one tile row per run (same box,
      // 256 x 2560 x 2048 + RoPE: 10.15 -> 9.85 us; 256 x 2048 x 8192:
      // 18.08 -> 17.17 us; four rows a run measured 9.98 and 17.15)
      case 2: return launch_tiles<64, 64, 32, 32, 4, 2, 1, 64, false, ROPE>(a, st);
      default: return launch_tiles<64, 32, 32, 32, 4, 2, 2, 64, false, ROPE>(a, st);
    }
  }
  // rows past M are not loaded (at M <= 16, 8 of every 12 load
  // instructions would only fetch zeros): M = 1 9.3 -> 8.8 us, M = 16
  // 9.8 -> 9.3 us for 6144 x 4096 weights. At M <= 16 a three-deep ring of
  // 512-deep stages keeps more of the weight stream in flight (M = 1
  // 8.75 -> 8.50 us, M = 16 9.23 -> 9.05 us; it loses at M = 32 and 64).
  // At M <= 32 one 32 x 32 tile of two K-splitting waves (KW = 2).
  // At M <= 8 (only the first 8-row A load of each stage fetches data) in
  // one round (a block per CU, LDS to spare) a four-deep ring keeps more of
  // the weight stream in flight (6144 x 4096 weights, ring depth 3 / 4 / 5
  // / 6: M = 1 7.16 / 6.64 / 6.74 / 7.01 us, M = 8 7.86 / 7.58 / 7.69 /
  // 7.83; M = 9 and 16 keep the three-deep ring, which a five-deep one did
  // not beat). Deeper rings at
  // M = 16, 32 and 64 (five, seven and six deep) and for the one-round
  // 64x64 plan measured level or slower (8.15 -> 8.17, 9.40 -> 9.46,
  // 11.27 -> 11.64; 256 x 2560 x 2048 8.73 -> 9.24 us).
  if (a.M <= 8 && a.K % 512 == 0 && (a.N + 31) / 32 <= device_cus())
    return launch_tiles<32, 32, 32, 32, 4, 1, 4, 16, false, ROPE, false, true, 2>(a, st);
  if (a.M <= 16 && a.K % 512 == 0) return launch_tiles<32, 32, 32, 32, 3, 1, 4, 16, false, ROPE, false, true, 2>(a, st);
  if (a.M <= 16) return launch_tiles<32, 32, 32, 32, 4, 1, 2, 16, false, ROPE, false, true, 2>(a, st);
  if (a.M <= 32) return launch_tiles<32, 32, 32, 32, 4, 1, 2, 32, false, ROPE, false, true, 2>(a, st);
  return launch_tiles<64, 32, 32, 32, 4, 1, 2, 64, false, ROPE, false, true>(a, st);
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
template <int AE, bool ROPE, bool WNT>
hipError_t launch_mx_narrow(const GemmArgs& a, hipStream_t st) {
  if (a.K % 1024 == 0) return launch_tiles<64, 32, 32, 32, 3, 1, 4, AE, false, ROPE, true, WNT>(a, st);
  if (a.K % 512 == 0) return launch_tiles<64, 32, 32, 32, 4, 1, 2, AE, false, ROPE, true, WNT>(a, st);
  return launch_tiles<64, 32, 32, 32, 7, 1, 1, AE, false, ROPE, true, WNT>(a, st);
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
    return launch_mx_narrow<64, ROPE, false>(a, st);
  }
  // one row of tiles: the weight stream is read once, non-temporally
  if (a.M <= 16) return launch_mx_narrow<16, ROPE, true>(a, st);
  if (a.M <= 32) return launch_mx_narrow<32, ROPE, true>(a, st);
  return launch_mx_narrow<64, ROPE, true>(a, st);
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

// GEGLU plans: chosen by plan_cost: 256x256 (M >= 512, gemm256_kernel),
// 128x128 of eight 32x64 waves, 64x64 of two 32x64 waves (also every
// M <= 64); a lane holds a gate column and its up column.
hipError_t launch_gemm_geglu(const GemmArgs& a, hipStream_t st) {
  if (a.M > 64) {
    const int cus = device_cus();
    const int64_t c256 = a.M >= 512 ? plan_cost(a, 256, 256, cus) : INT64_MAX;
    const int64_t c128 = plan_cost(a, 128, 128, cus), c64 = plan_cost(a, 64, 64, cus);
    if (c256 < c128 && c256 < c64)
      return launch_256<true, false>(a, st);
    if (c128 < c64) return launch_tiles<128, 128, 32, 64, 3, 2, 1, 128, true>(a, st);
  }
  return launch_tiles<64, 64, 32, 64, 4, 1, 1, 64, true>(a, st);
}

}  // namespace frt
