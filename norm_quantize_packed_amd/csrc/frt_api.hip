// C ABI of the frt library: argument validation, refusal reasons, dispatch.
//
// Every check runs on the host before any launch, so a refused call leaves
// all buffers untouched. The contracts follow the pages' own refusals
// (flashrt-structures 0.2.0): the per-token-table producer's SUPPORT
// envelope (6 chunks, D in [512, 16384], even) in
// impls/modnorm_qkv_chain/fp8_ptok_table.py `bind_block_seam`; the
// projection envelope (K in [512, 16384]) of impls/linear_proj/
// fp8_static.py; the row-capacity contract and the aliasing checks of
// impls/qkv_pack/fp8_static.py (`PackedLinear`, `alias_stash`).
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "frt_internal.h"

namespace {

thread_local char g_err[512] = "";

int refuse(int code, const char* fmt, ...) {
  char msg[448];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  snprintf(g_err, sizeof g_err, "refused: %s", msg);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return FRT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return refuse(FRT_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// [lo, hi) byte range covered by a [rows, cols] matrix with row stride ld
struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  if (p == nullptr || rows <= 0) return Range{0, 0};
  const uintptr_t lo = (uintptr_t)p;
  return Range{lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * esize)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Do two [rows, cols] matrices with row stride ld (elements of esize bytes)
// share an element? Exact when both use the same stride (columns of one
// buffer handed to different splits, rows interleaved); otherwise the
// conservative byte-span test.
bool overlap_mat(const void* p, int64_t rp, int64_t cp, const void* q, int64_t rq, int64_t cq,
                 int64_t ld, int64_t esize) {
  if (p == nullptr || q == nullptr || rp <= 0 || rq <= 0) return false;
  const int64_t db = (int64_t)((intptr_t)q - (intptr_t)p);
  if (db % esize != 0 || cp > ld || cq > ld)
    return overlap(span(p, rp, cp, ld, esize), span(q, rq, cq, ld, esize));
  const int64_t d = db / esize;  // q = p + d elements
  int64_t qd = d / ld, r = d % ld;
  if (r < 0) { r += ld; qd -= 1; }
  // element (i, c1) of p equals (j, c2) of q iff (i - j) * ld + (c1 - c2) = d
  const bool same_row = r < cp && qd > -rq && qd < rp;            // i - j = qd
  const bool next_row = (ld - r) < cq && qd + 1 > -rq && qd + 1 < rp;  // i - j = qd + 1
  return same_row || next_row;
}

constexpr int64_t kDMin = 512, kDMax = 16384;

}  // namespace

extern "C" {

const char* frt_last_error(void) { return g_err; }

int frt_abi_version(void) { return 1; }

int frt_ada_norm_quant_fp8(void* stream, int64_t M, int64_t D, const uint16_t* residual,
                           int64_t ld_res, const uint16_t* x, int64_t ld_x, const uint16_t* gate,
                           int64_t ld_gate, const uint16_t* weight, const uint16_t* mod,
                           int64_t ld_mod, const float* act_scale, float eps,
                           uint16_t* residual_out, int64_t ld_rout, uint8_t* out_fp8,
                           int64_t ld_out, uint16_t* gate_out, int64_t ld_gout, float* y_f32,
                           int64_t ld_y, float* amax_out) {
  if (M < 0) return refuse(FRT_E_INVALID, "ada_norm: M=%lld < 0", (long long)M);
  if (D < kDMin || D > kDMax || D % 2)
    return refuse(FRT_E_INVALID, "ada_norm: D=%lld outside [512, 16384] or odd", (long long)D);
  if (M > (int64_t)0x7fffffff) return refuse(FRT_E_UNSUPPORTED, "ada_norm: M too large");
  if (residual == nullptr || mod == nullptr)
    return refuse(FRT_E_INVALID, "ada_norm: residual and mod are required");
  if (ld_res < D) return refuse(FRT_E_INVALID, "ada_norm: ld_res < D");
  if (x != nullptr && ld_x < D) return refuse(FRT_E_INVALID, "ada_norm: ld_x < D");
  if (gate != nullptr && ld_gate != 0 && ld_gate < D)
    return refuse(FRT_E_INVALID, "ada_norm: ld_gate must be 0 (broadcast) or >= D");
  if (ld_mod != 0 && ld_mod < 3 * D)
    return refuse(FRT_E_INVALID, "ada_norm: ld_mod must be 0 (broadcast) or >= 3*D");
  if (out_fp8 != nullptr && act_scale == nullptr)
    return refuse(FRT_E_INVALID, "ada_norm: out_fp8 needs act_scale");
  if (residual_out != nullptr && ld_rout < D) return refuse(FRT_E_INVALID, "ada_norm: ld_rout < D");
  if (out_fp8 != nullptr && ld_out < D) return refuse(FRT_E_INVALID, "ada_norm: ld_out < D");
  if (gate_out != nullptr && ld_gout < D) return refuse(FRT_E_INVALID, "ada_norm: ld_gout < D");
  if (y_f32 != nullptr && ld_y < D) return refuse(FRT_E_INVALID, "ada_norm: ld_y < D");
  if (out_fp8 == nullptr && residual_out == nullptr && gate_out == nullptr && y_f32 == nullptr &&
      amax_out == nullptr)
    return refuse(FRT_E_INVALID, "ada_norm: no output requested");
  if (M == 0) return ok();

  // aliasing: residual_out may be residual itself (same ld); nothing else
  const int64_t mrows = ld_mod ? M : 1, grows = ld_gate ? M : 1;
  const Range in[] = {span(residual, M, D, ld_res, 2), span(x, M, D, ld_x, 2),
                      span(gate, grows, D, ld_gate ? ld_gate : D, 2), span(weight, 1, D, D, 2),
                      span(mod, mrows, 3 * D, ld_mod ? ld_mod : 3 * D, 2),
                      span(act_scale, 1, 1, 1, 4)};
  const Range outs[] = {span(residual_out, M, D, ld_rout, 2), span(out_fp8, M, D, ld_out, 1),
                        span(gate_out, M, D, ld_gout, 2), span(y_f32, M, D, ld_y, 4),
                        span(amax_out, 1, 1, 1, 4)};
  const bool inplace = residual_out != nullptr && residual_out == residual && ld_rout == ld_res;
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 6; ++i) {
      if (o == 0 && i == 0 && inplace) continue;
      if (overlap(outs[o], in[i]))
        return refuse(FRT_E_INVALID, "ada_norm: output %d overlaps input %d (only an exact in-place residual is allowed)", o, i);
    }
    for (int p = o + 1; p < 5; ++p)
      if (overlap(outs[o], outs[p])) return refuse(FRT_E_INVALID, "ada_norm: outputs %d and %d overlap", o, p);
  }

  const bool vec8 = D % 8 == 0 && aligned(residual, 16) && ld_res % 8 == 0 &&
                    (x == nullptr || (aligned(x, 16) && ld_x % 8 == 0)) &&
                    (gate == nullptr || (aligned(gate, 16) && ld_gate % 8 == 0)) &&
                    (weight == nullptr || aligned(weight, 16)) && aligned(mod, 16) && ld_mod % 8 == 0 &&
                    (residual_out == nullptr || (aligned(residual_out, 16) && ld_rout % 8 == 0)) &&
                    (out_fp8 == nullptr || (aligned(out_fp8, 8) && ld_out % 8 == 0)) &&
                    (gate_out == nullptr || (aligned(gate_out, 16) && ld_gout % 8 == 0)) &&
                    (y_f32 == nullptr || (aligned(y_f32, 16) && ld_y % 4 == 0));
  if (!vec8) {
    const bool a4 = aligned(residual, 4) && ld_res % 2 == 0 && (x == nullptr || (aligned(x, 4) && ld_x % 2 == 0)) &&
                    (gate == nullptr || (aligned(gate, 4) && ld_gate % 2 == 0)) &&
                    (weight == nullptr || aligned(weight, 4)) && aligned(mod, 4) && ld_mod % 2 == 0 &&
                    (residual_out == nullptr || (aligned(residual_out, 4) && ld_rout % 2 == 0)) &&
                    (out_fp8 == nullptr || (aligned(out_fp8, 2) && ld_out % 2 == 0)) &&
                    (gate_out == nullptr || (aligned(gate_out, 4) && ld_gout % 2 == 0)) &&
                    (y_f32 == nullptr || (aligned(y_f32, 8) && ld_y % 2 == 0));
    if (!a4) return refuse(FRT_E_INVALID, "ada_norm: pointers/strides must be at least 4-byte aligned (2 elements)");
  }
  frt::AdaArgs a{residual, ld_res, x, ld_x, gate, ld_gate, weight, mod, ld_mod,
                 act_scale, eps, residual_out, ld_rout, out_fp8, ld_out, gate_out, ld_gout,
                 y_f32, ld_y, amax_out, M, (int)D};
  if (x == nullptr || gate == nullptr) {
    a.x = nullptr;
    a.gate = nullptr;
  }
  return hip_status(frt::launch_ada_norm(a, vec8, (hipStream_t)stream), "ada_norm launch");
}

int frt_ptok_table_norm_quant_fp8(void* stream, int64_t R, int64_t D, int C, const uint16_t* x,
                                  int64_t ld_x, const uint16_t* temb, int64_t ld_temb,
                                  const float* table, const float* act_scale, int shift_idx,
                                  int scale_idx, float eps, uint8_t* out_fp8, int64_t ld_out,
                                  float* y_f32, int64_t ld_y, float* amax_out) {
  if (R < 0) return refuse(FRT_E_INVALID, "ptok_norm: R=%lld < 0", (long long)R);
  if (C != 6) return refuse(FRT_E_INVALID, "ptok_norm: %d-chunk table; the 6-chunk layout is served", C);
  if (D < kDMin || D > kDMax || D % 2)
    return refuse(FRT_E_INVALID, "ptok_norm: D=%lld outside [512, 16384] or odd", (long long)D);
  if (R > (int64_t)0x7fffffff) return refuse(FRT_E_UNSUPPORTED, "ptok_norm: R too large");
  if (shift_idx < 0 || shift_idx >= C || scale_idx < 0 || scale_idx >= C)
    return refuse(FRT_E_INVALID, "ptok_norm: chunk index outside [0, %d)", C);
  if (x == nullptr || temb == nullptr || table == nullptr)
    return refuse(FRT_E_INVALID, "ptok_norm: x, temb and table are required");
  if (ld_x < D) return refuse(FRT_E_INVALID, "ptok_norm: ld_x < D");
  if (ld_temb < (int64_t)C * D) return refuse(FRT_E_INVALID, "ptok_norm: ld_temb < C*D");
  if (out_fp8 != nullptr && act_scale == nullptr)
    return refuse(FRT_E_INVALID, "ptok_norm: out_fp8 needs act_scale");
  if (out_fp8 != nullptr && ld_out < D) return refuse(FRT_E_INVALID, "ptok_norm: ld_out < D");
  if (y_f32 != nullptr && ld_y < D) return refuse(FRT_E_INVALID, "ptok_norm: ld_y < D");
  if (out_fp8 == nullptr && y_f32 == nullptr && amax_out == nullptr)
    return refuse(FRT_E_INVALID, "ptok_norm: no output requested");
  if (R == 0) return ok();
  const Range in[] = {span(x, R, D, ld_x, 2), span(temb, R, (int64_t)C * D, ld_temb, 2),
                      span(table, C, D, D, 4), span(act_scale, 1, 1, 1, 4)};
  const Range outs[] = {span(out_fp8, R, D, ld_out, 1), span(y_f32, R, D, ld_y, 4), span(amax_out, 1, 1, 1, 4)};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlap(outs[o], in[i])) return refuse(FRT_E_INVALID, "ptok_norm: output %d overlaps input %d", o, i);
    for (int p = o + 1; p < 3; ++p)
      if (overlap(outs[o], outs[p])) return refuse(FRT_E_INVALID, "ptok_norm: outputs %d and %d overlap", o, p);
  }
  const bool vec8 = D % 8 == 0 && aligned(x, 16) && ld_x % 8 == 0 && aligned(temb, 16) && ld_temb % 8 == 0 &&
                    aligned(table, 16) && (out_fp8 == nullptr || (aligned(out_fp8, 8) && ld_out % 8 == 0)) &&
                    (y_f32 == nullptr || (aligned(y_f32, 16) && ld_y % 4 == 0));
  if (!vec8) {
    const bool a4 = aligned(x, 4) && ld_x % 2 == 0 && aligned(temb, 4) && ld_temb % 2 == 0 && aligned(table, 8) &&
                    (out_fp8 == nullptr || (aligned(out_fp8, 2) && ld_out % 2 == 0)) &&
                    (y_f32 == nullptr || (aligned(y_f32, 8) && ld_y % 2 == 0));
    if (!a4) return refuse(FRT_E_INVALID, "ptok_norm: pointers/strides must be at least 4-byte aligned (2 elements)");
  }
  frt::PtokArgs a{x, ld_x, temb, ld_temb, table, act_scale, eps, shift_idx, scale_idx,
                  out_fp8, ld_out, y_f32, ld_y, amax_out, R, (int)D};
  return hip_status(frt::launch_ptok_norm(a, vec8, (hipStream_t)stream), "ptok_norm launch");
}

int frt_pack_weights_fp8(void* stream, int n_sib, const int64_t* N_i, int64_t K,
                         const uint16_t* const* W_i, const uint16_t* const* b_i, uint8_t* W8,
                         float* w_scale, uint16_t* bias_cat) {
  if (n_sib < 1 || n_sib > FRT_MAX_SPLITS)
    return refuse(FRT_E_INVALID, "pack: n_sib=%d outside [1, %d]", n_sib, FRT_MAX_SPLITS);
  if (N_i == nullptr || W_i == nullptr || W8 == nullptr || w_scale == nullptr)
    return refuse(FRT_E_INVALID, "pack: N_i, W_i, W8 and w_scale are required");
  if (K < 1) return refuse(FRT_E_INVALID, "pack: K=%lld < 1", (long long)K);
  frt::PackSib sibs[FRT_MAX_SPLITS];
  int64_t rows = 0;
  for (int i = 0; i < n_sib; ++i) {
    if (N_i[i] < 1) return refuse(FRT_E_INVALID, "pack: N_%d=%lld < 1", i, (long long)N_i[i]);
    if (W_i[i] == nullptr) return refuse(FRT_E_INVALID, "pack: W_%d is NULL", i);
    if (!aligned(W_i[i], 2)) return refuse(FRT_E_INVALID, "pack: W_%d misaligned", i);
    sibs[i].w = W_i[i];
    sibs[i].b = b_i != nullptr ? b_i[i] : nullptr;
    sibs[i].rows = N_i[i];
    sibs[i].row_off = rows;
    sibs[i].elems = N_i[i] * K;
    sibs[i].dst_off = rows * K;
    rows += N_i[i];
  }
  if (rows * K > ((int64_t)1 << 40)) return refuse(FRT_E_UNSUPPORTED, "pack: matrix too large");
  const Range w8r = span(W8, rows, K, K, 1), sr = span(w_scale, 1, 1, 1, 4), br = span(bias_cat, 1, rows, rows, 2);
  if (overlap(w8r, sr) || overlap(w8r, br) || overlap(sr, br)) return refuse(FRT_E_INVALID, "pack: outputs overlap");
  for (int i = 0; i < n_sib; ++i) {
    const Range wr = span(sibs[i].w, sibs[i].rows, K, K, 2);
    const Range bb = span(sibs[i].b, 1, sibs[i].rows, sibs[i].rows, 2);
    if (overlap(wr, w8r) || overlap(wr, sr) || overlap(wr, br) || overlap(bb, w8r) || overlap(bb, sr) ||
        overlap(bb, br))
      return refuse(FRT_E_INVALID, "pack: sibling %d overlaps an output", i);
  }
  return hip_status(frt::launch_pack(sibs, n_sib, K, W8, w_scale, bias_cat, (hipStream_t)stream), "pack launch");
}

size_t frt_packed_gemm_fp8_workspace_size(int64_t M, int64_t N_total, int64_t K) {
  if (M <= 0 || N_total <= 0 || K <= 0) return 0;
  return frt::gemm_workspace_bytes(M, N_total, K);
}

}  // extern "C"

namespace {

// Every check of the packed split GEMM's contract (shapes, strides,
// alignment, splits, workspace, overlaps) and its kernel arguments; no
// launch. FRT_OK with a.M == 0 means there is nothing to run.
// kb: operand bytes per row (K for FP8, K / 2 for MXFP4 codes).
int gemm_prepare(int64_t M, int64_t K, int64_t kb, const uint8_t* x8, int64_t ld_x, const uint8_t* W8,
                 int64_t N_total,
                 const float* act_scale, const float* w_scale, const uint16_t* bias_cat, int n_split,
                 const int64_t* split_n, void* const* out, const int64_t* ld_out, int out_dtype, void* workspace,
                 size_t ws_bytes, frt::GemmArgs& a) {
  if (M < 0) return refuse(FRT_E_INVALID, "gemm: M=%lld < 0", (long long)M);
  if (K < 512 || K > 16384) return refuse(FRT_E_INVALID, "gemm: K=%lld outside [512, 16384]", (long long)K);
  if (K % 16) return refuse(FRT_E_UNSUPPORTED, "gemm: K=%lld not a multiple of 16", (long long)K);
  if (N_total < 1) return refuse(FRT_E_INVALID, "gemm: N_total < 1");
  if (M > (1 << 24) || N_total > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "gemm: M or N_total too large");
  if (x8 == nullptr || W8 == nullptr || act_scale == nullptr || w_scale == nullptr)
    return refuse(FRT_E_INVALID, "gemm: x8, W8, act_scale and w_scale are required");
  if (ld_x < kb || ld_x % 16) return refuse(FRT_E_INVALID, "gemm: ld_x must be >= the row bytes and a multiple of 16");
  if (!aligned(x8, 16) || !aligned(W8, 16)) return refuse(FRT_E_INVALID, "gemm: x8 and W8 must be 16-byte aligned");
  if ((M - 1) * ld_x + kb > (int64_t)0x7fffffff || N_total * kb > (int64_t)0x7fffffff)
    return refuse(FRT_E_UNSUPPORTED, "gemm: operand larger than 2 GiB");
  if (out_dtype != 0 && out_dtype != 1) return refuse(FRT_E_INVALID, "gemm: out_dtype must be 0 (bf16) or 1 (fp32)");
  if (n_split < 1 || n_split > FRT_MAX_SPLITS)
    return refuse(FRT_E_INVALID, "gemm: n_split=%d outside [1, %d]", n_split, FRT_MAX_SPLITS);
  if (split_n == nullptr || out == nullptr || ld_out == nullptr)
    return refuse(FRT_E_INVALID, "gemm: split_n, out and ld_out are required");
  const int64_t es = out_dtype ? 4 : 2;
  a = frt::GemmArgs{};
  int64_t tot = 0;
  for (int s = 0; s < n_split; ++s) {
    if (split_n[s] < 1) return refuse(FRT_E_INVALID, "gemm: split %d has width %lld < 1", s, (long long)split_n[s]);
    if (out[s] == nullptr) return refuse(FRT_E_INVALID, "gemm: out[%d] is NULL", s);
    if (ld_out[s] < split_n[s]) return refuse(FRT_E_INVALID, "gemm: ld_out[%d] < split width", s);
    if (!aligned(out[s], (size_t)es)) return refuse(FRT_E_INVALID, "gemm: out[%d] misaligned", s);
    a.sp.ptr[s] = out[s];
    a.sp.ld[s] = ld_out[s];
    a.sp.off[s] = (int)tot;
    tot += split_n[s];
  }
  if (tot != N_total)
    return refuse(FRT_E_INVALID, "gemm: splits sum to %lld, N_total is %lld", (long long)tot, (long long)N_total);
  a.sp.off[n_split] = (int)tot;
  for (int s = n_split + 1; s <= FRT_MAX_SPLITS; ++s) a.sp.off[s] = (int)tot;
  a.sp.n = n_split;
  const size_t need = frt::gemm_workspace_bytes(M, N_total, K);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return refuse(FRT_E_INVALID, "gemm: workspace of %zu bytes required", need);
  if (M == 0) return FRT_OK;
  // outputs must not overlap each other or the inputs
  const Range xin = span(x8, M, kb, ld_x, 1), win = span(W8, N_total, kb, kb, 1),
              bin = span(bias_cat, 1, N_total, N_total, 2), sa = span(act_scale, 1, 1, 1, 4),
              sw = span(w_scale, 1, 1, 1, 4), wsr = span(workspace, 1, (int64_t)need, (int64_t)need, 1);
  for (int s = 0; s < n_split; ++s) {
    const Range o = span(out[s], M, split_n[s], ld_out[s], es);
    if (overlap(o, xin) || overlap(o, win) || overlap(o, bin) || overlap(o, sa) || overlap(o, sw) || overlap(o, wsr))
      return refuse(FRT_E_INVALID, "gemm: output %d overlaps an input or the workspace", s);
    for (int t = s + 1; t < n_split; ++t) {
      const bool ov = ld_out[s] == ld_out[t]
                          ? overlap_mat(out[s], M, split_n[s], out[t], M, split_n[t], ld_out[s], es)
                          : overlap(o, span(out[t], M, split_n[t], ld_out[t], es));
      if (ov) return refuse(FRT_E_INVALID, "gemm: outputs %d and %d overlap", s, t);
    }
  }
  a.x = x8;
  a.ld_x = ld_x;
  a.w = W8;
  a.act_scale = act_scale;
  a.w_scale = w_scale;
  a.bias = bias_cat;
  a.M = (int)M;
  a.N = (int)N_total;
  a.K = (int)K;
  a.out_f32 = out_dtype;
  a.vec_out = out_dtype == 0;
  for (int s = 0; s < n_split; ++s)
    if (split_n[s] % 8 || ld_out[s] % 8 || !aligned(out[s], 16)) a.vec_out = 0;
  return FRT_OK;
}

}  // namespace

extern "C" {

int frt_packed_gemm_fp8_split(void* stream, int64_t M, int64_t K, const uint8_t* x8, int64_t ld_x,
                              const uint8_t* W8, int64_t N_total, const float* act_scale,
                              const float* w_scale, const uint16_t* bias_cat, int n_split,
                              const int64_t* split_n, void* const* out, const int64_t* ld_out,
                              int out_dtype, void* workspace, size_t ws_bytes) {
  frt::GemmArgs a;
  const int rc = gemm_prepare(M, K, K, x8, ld_x, W8, N_total, act_scale, w_scale, bias_cat, n_split, split_n, out,
                              ld_out, out_dtype, workspace, ws_bytes, a);
  if (rc != FRT_OK) return rc;
  if (M == 0) return ok();
  return hip_status(frt::launch_gemm(a, (hipStream_t)stream), "gemm launch");
}

int frt_geglu_quant_fp8(void* stream, int64_t M, int64_t H, const uint16_t* gu, int64_t ld_gu,
                        const float* act_scale, uint8_t* out_fp8, int64_t ld_out, float* y_f32,
                        int64_t ld_y, float* amax_out) {
  if (M < 0) return refuse(FRT_E_INVALID, "geglu: M=%lld < 0", (long long)M);
  if (H < 1 || H > (1 << 24)) return refuse(FRT_E_INVALID, "geglu: H=%lld outside [1, 2^24]", (long long)H);
  if (gu == nullptr) return refuse(FRT_E_INVALID, "geglu: gu is required");
  if (ld_gu < 2 * H) return refuse(FRT_E_INVALID, "geglu: ld_gu < 2*H");
  if (out_fp8 != nullptr && act_scale == nullptr) return refuse(FRT_E_INVALID, "geglu: out_fp8 needs act_scale");
  if (out_fp8 != nullptr && ld_out < H) return refuse(FRT_E_INVALID, "geglu: ld_out < H");
  if (y_f32 != nullptr && ld_y < H) return refuse(FRT_E_INVALID, "geglu: ld_y < H");
  if (out_fp8 == nullptr && y_f32 == nullptr && amax_out == nullptr)
    return refuse(FRT_E_INVALID, "geglu: no output requested");
  if (!aligned(gu, 2) || (y_f32 != nullptr && !aligned(y_f32, 4)))
    return refuse(FRT_E_INVALID, "geglu: gu (y_f32) must be 2 (4)-byte aligned");
  if (M == 0) return ok();
  const Range in[] = {span(gu, M, 2 * H, ld_gu, 2), span(act_scale, 1, 1, 1, 4)};
  const Range outs[] = {span(out_fp8, M, H, ld_out, 1), span(y_f32, M, H, ld_y, 4), span(amax_out, 1, 1, 1, 4)};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 2; ++i)
      if (overlap(outs[o], in[i])) return refuse(FRT_E_INVALID, "geglu: output %d overlaps input %d", o, i);
    for (int p = o + 1; p < 3; ++p)
      if (overlap(outs[o], outs[p])) return refuse(FRT_E_INVALID, "geglu: outputs %d and %d overlap", o, p);
  }
  const bool vec8 = H % 8 == 0 && aligned(gu, 16) && ld_gu % 8 == 0 &&
                    (out_fp8 == nullptr || (aligned(out_fp8, 8) && ld_out % 8 == 0)) &&
                    (y_f32 == nullptr || (aligned(y_f32, 16) && ld_y % 4 == 0));
  frt::GegluArgs a{gu, ld_gu, act_scale, out_fp8, ld_out, y_f32, ld_y, amax_out, M, (int)H};
  return hip_status(frt::launch_geglu(a, vec8 ? 8 : 1, (hipStream_t)stream), "geglu launch");
}

namespace {

// Shared contract of the two MXFP4 quantisers from bf16: `cols` input
// columns per row (2H for the GEGLU form), H output columns.
int mx_quant(const char* who, void* stream, int64_t M, int64_t H, int64_t cols, const uint16_t* x, int64_t ld_x,
             uint8_t* out_fp4, int64_t ld_out, uint8_t* out_scale, int64_t ld_sc, bool glu) {
  if (M < 0) return refuse(FRT_E_INVALID, "%s: M=%lld < 0", who, (long long)M);
  if (H < 256 || cols > (1 << 24) || H % 256)
    return refuse(FRT_E_INVALID, "%s: width %lld must be a multiple of 256 (at most 2^24 input columns)", who,
                  (long long)H);
  if (x == nullptr || out_fp4 == nullptr || out_scale == nullptr)
    return refuse(FRT_E_INVALID, "%s: input, out_fp4 and out_scale are required", who);
  if (ld_x < cols || ld_x % 8 || !aligned(x, 16))
    return refuse(FRT_E_INVALID, "%s: input 16-byte aligned with a row stride >= its columns and a multiple of 8",
                  who);
  if (ld_out < H / 2 || ld_out % 4 || !aligned(out_fp4, 4))
    return refuse(FRT_E_INVALID, "%s: out_fp4 4-byte aligned, ld_out >= H/2 and a multiple of 4", who);
  if (ld_sc < 8 * M) return refuse(FRT_E_INVALID, "%s: ld_sc (the scale run stride) < 8*M", who);
  if (M == 0) return ok();
  const Range in = span(x, M, cols, ld_x, 2), o = span(out_fp4, M, H / 2, ld_out, 1),
              sc = span(out_scale, H / 256, 8 * M, ld_sc, 1);
  if (overlap(o, in) || overlap(sc, in) || overlap(o, sc))
    return refuse(FRT_E_INVALID, "%s: outputs overlap the input or each other", who);
  frt::GegluArgs a{};
  a.gu = x;
  a.ld_gu = ld_x;
  a.out = out_fp4;
  a.ld_out = ld_out;
  a.M = M;
  a.H = (int)H;
  a.sc = out_scale;
  a.ld_sc = ld_sc;
  return hip_status(frt::launch_mx_quant(a, glu, (hipStream_t)stream), who);
}

}  // namespace

int frt_quantize_mxfp4(void* stream, int64_t M, int64_t D, const uint16_t* x, int64_t ld_x, uint8_t* out_fp4,
                       int64_t ld_out, uint8_t* out_scale, int64_t ld_sc) {
  return mx_quant("quantize_mxfp4", stream, M, D, D, x, ld_x, out_fp4, ld_out, out_scale, ld_sc, false);
}

int frt_geglu_quant_mxfp4(void* stream, int64_t M, int64_t H, const uint16_t* gu, int64_t ld_gu, uint8_t* out_fp4,
                          int64_t ld_out, uint8_t* out_scale, int64_t ld_sc) {
  return mx_quant("geglu_mxfp4", stream, M, H, 2 * H, gu, ld_gu, out_fp4, ld_out, out_scale, ld_sc, true);
}

int frt_packed_gemm_fp8_geglu_quant(void* stream, int64_t M, int64_t K, const uint8_t* x8, int64_t ld_x,
                                    const uint8_t* W8, int64_t H, const float* act_scale,
                                    const float* w_scale, const uint16_t* bias_cat,
                                    const float* out_scale, uint8_t* out_fp8, int64_t ld_out) {
  if (M < 0) return refuse(FRT_E_INVALID, "gemm_geglu: M=%lld < 0", (long long)M);
  if (K < 512 || K > 16384) return refuse(FRT_E_INVALID, "gemm_geglu: K=%lld outside [512, 16384]", (long long)K);
  if (K % 16) return refuse(FRT_E_UNSUPPORTED, "gemm_geglu: K=%lld not a multiple of 16", (long long)K);
  if (H < 1) return refuse(FRT_E_INVALID, "gemm_geglu: H < 1");
  if (M > (1 << 24) || 2 * H > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "gemm_geglu: M or 2H too large");
  if (x8 == nullptr || W8 == nullptr || act_scale == nullptr || w_scale == nullptr || out_scale == nullptr ||
      out_fp8 == nullptr)
    return refuse(FRT_E_INVALID, "gemm_geglu: x8, W8, act_scale, w_scale, out_scale and out_fp8 are required");
  if (ld_x < K || ld_x % 16) return refuse(FRT_E_INVALID, "gemm_geglu: ld_x must be >= K and a multiple of 16");
  if (!aligned(x8, 16) || !aligned(W8, 16))
    return refuse(FRT_E_INVALID, "gemm_geglu: x8 and W8 must be 16-byte aligned");
  if ((M - 1) * ld_x + K > (int64_t)0x7fffffff || 2 * H * K > (int64_t)0x7fffffff)
    return refuse(FRT_E_UNSUPPORTED, "gemm_geglu: operand larger than 2 GiB");
  if (ld_out < H) return refuse(FRT_E_INVALID, "gemm_geglu: ld_out < H");
  if (M == 0) return ok();
  const Range o = span(out_fp8, M, H, ld_out, 1);
  const Range in[] = {span(x8, M, K, ld_x, 1), span(W8, 2 * H, K, K, 1), span(bias_cat, 1, 2 * H, 2 * H, 2),
                      span(act_scale, 1, 1, 1, 4), span(w_scale, 1, 1, 1, 4), span(out_scale, 1, 1, 1, 4)};
  for (int i = 0; i < 6; ++i)
    if (overlap(o, in[i])) return refuse(FRT_E_INVALID, "gemm_geglu: out_fp8 overlaps input %d", i);
  frt::GemmArgs a{};
  a.x = x8;
  a.ld_x = ld_x;
  a.w = W8;
  a.act_scale = act_scale;
  a.w_scale = w_scale;
  a.bias = bias_cat;
  a.M = (int)M;
  a.N = (int)(2 * H);
  a.K = (int)K;
  a.H = (int)H;
  a.q8 = out_fp8;
  a.ld_q8 = ld_out;
  a.q_scale = out_scale;
  return hip_status(frt::launch_gemm_geglu(a, (hipStream_t)stream), "gemm_geglu launch");
}

int frt_quantize_fp8_static(void* stream, int64_t M, int64_t D, const uint16_t* x, int64_t ld_x,
                            const float* act_scale, uint8_t* out_fp8, int64_t ld_out, float* amax_out) {
  if (M < 0) return refuse(FRT_E_INVALID, "quantize: M=%lld < 0", (long long)M);
  if (D < 1 || D > (1 << 24)) return refuse(FRT_E_INVALID, "quantize: D=%lld outside [1, 2^24]", (long long)D);
  if (x == nullptr) return refuse(FRT_E_INVALID, "quantize: x is required");
  if (ld_x < D) return refuse(FRT_E_INVALID, "quantize: ld_x < D");
  if (out_fp8 != nullptr && act_scale == nullptr) return refuse(FRT_E_INVALID, "quantize: out_fp8 needs act_scale");
  if (out_fp8 != nullptr && ld_out < D) return refuse(FRT_E_INVALID, "quantize: ld_out < D");
  if (out_fp8 == nullptr && amax_out == nullptr) return refuse(FRT_E_INVALID, "quantize: no output requested");
  if (!aligned(x, 2)) return refuse(FRT_E_INVALID, "quantize: x misaligned");
  if (M == 0) return ok();
  const Range in[] = {span(x, M, D, ld_x, 2), span(act_scale, 1, 1, 1, 4)};
  const Range outs[] = {span(out_fp8, M, D, ld_out, 1), span(amax_out, 1, 1, 1, 4)};
  for (int o = 0; o < 2; ++o)
    for (int i = 0; i < 2; ++i)
      if (overlap(outs[o], in[i])) return refuse(FRT_E_INVALID, "quantize: output %d overlaps input %d", o, i);
  if (overlap(outs[0], outs[1])) return refuse(FRT_E_INVALID, "quantize: outputs overlap");
  const bool vec8 = D % 8 == 0 && aligned(x, 16) && ld_x % 8 == 0 &&
                    (out_fp8 == nullptr || (aligned(out_fp8, 8) && ld_out % 8 == 0));
  frt::GegluArgs a{x, ld_x, act_scale, out_fp8, ld_out, nullptr, 0, amax_out, M, (int)D};
  return hip_status(frt::launch_quant(a, vec8 ? 8 : 1, (hipStream_t)stream), "quantize launch");
}

int frt_packed_gemm_bf16in_split(void* stream, int64_t M, int64_t K, const uint16_t* x, int64_t ld_x, uint8_t* x8,
                                 int64_t ld_x8, const uint8_t* W8, int64_t N_total, const float* act_scale,
                                 const float* w_scale, const uint16_t* bias_cat, int n_split,
                                 const int64_t* split_n, void* const* out, const int64_t* ld_out, int out_dtype,
                                 void* workspace, size_t ws_bytes) {
  if (x == nullptr || x8 == nullptr) return refuse(FRT_E_INVALID, "gemm_bf16in: x and x8 are required");
  if (ld_x < K) return refuse(FRT_E_INVALID, "gemm_bf16in: ld_x < K");
  if (!aligned(x, 2)) return refuse(FRT_E_INVALID, "gemm_bf16in: x misaligned");
  // the GEMM's whole contract on the FP8 operand the call writes
  frt::GemmArgs a;
  const int rc = gemm_prepare(M, K, K, x8, ld_x8, W8, N_total, act_scale, w_scale, bias_cat, n_split, split_n, out,
                              ld_out, out_dtype, workspace, ws_bytes, a);
  if (rc != FRT_OK) return rc;
  if (M == 0) return ok();
  const Range xr = span(x, M, K, ld_x, 2), x8r = span(x8, M, K, ld_x8, 1);
  if (overlap(x8r, xr) || overlap(x8r, span(W8, N_total, K, K, 1)) || overlap(x8r, span(act_scale, 1, 1, 1, 4)) ||
      overlap(x8r, span(w_scale, 1, 1, 1, 4)) || overlap(x8r, span(bias_cat, 1, N_total, N_total, 2)))
    return refuse(FRT_E_INVALID, "gemm_bf16in: x8 overlaps an input");
  for (int s = 0; s < n_split; ++s) {
    const Range o = span(out[s], M, split_n[s], ld_out[s], out_dtype ? 4 : 2);
    if (overlap(o, xr) || overlap(o, x8r)) return refuse(FRT_E_INVALID, "gemm_bf16in: output %d overlaps x or x8", s);
  }
  const bool vec8 = K % 8 == 0 && aligned(x, 16) && ld_x % 8 == 0;  // x8: 16-byte aligned, ld % 16 (GEMM contract)
  frt::GegluArgs q{x, ld_x, act_scale, x8, ld_x8, nullptr, 0, nullptr, M, (int)K};
  const hipError_t e = frt::launch_quant(q, vec8 ? 8 : 1, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "gemm_bf16in quantize launch");
  return hip_status(frt::launch_gemm(a, (hipStream_t)stream), "gemm_bf16in launch");
}

int frt_pack_weights_mxfp4(void* stream, int n_sib, const int64_t* N_i, int64_t K, const uint16_t* const* W_i,
                           const uint16_t* const* b_i, uint8_t* W4, uint8_t* S4, uint16_t* bias_cat) {
  if (n_sib < 1 || n_sib > FRT_MAX_SPLITS)
    return refuse(FRT_E_INVALID, "pack_mxfp4: n_sib=%d outside [1, %d]", n_sib, FRT_MAX_SPLITS);
  if (N_i == nullptr || W_i == nullptr || W4 == nullptr || S4 == nullptr)
    return refuse(FRT_E_INVALID, "pack_mxfp4: N_i, W_i, W4 and S4 are required");
  if (K < 512 || K > 16384 || K % 256)
    return refuse(FRT_E_INVALID, "pack_mxfp4: K=%lld must be a multiple of 256 in [512, 16384]", (long long)K);
  if (!aligned(W4, 4)) return refuse(FRT_E_INVALID, "pack_mxfp4: W4 must be 4-byte aligned");
  frt::PackSib sibs[FRT_MAX_SPLITS];
  int64_t rows = 0;
  for (int i = 0; i < n_sib; ++i) {
    if (N_i[i] < 1) return refuse(FRT_E_INVALID, "pack_mxfp4: N_%d=%lld < 1", i, (long long)N_i[i]);
    if (W_i[i] == nullptr || !aligned(W_i[i], 16))
      return refuse(FRT_E_INVALID, "pack_mxfp4: W_%d must be 16-byte aligned", i);
    sibs[i].w = W_i[i];
    sibs[i].b = b_i != nullptr ? b_i[i] : nullptr;
    sibs[i].rows = N_i[i];
    sibs[i].row_off = rows;
    sibs[i].elems = N_i[i] * K;
    sibs[i].dst_off = rows * (K / 2);
    rows += N_i[i];
  }
  if (rows > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "pack_mxfp4: too many rows");
  const Range w4r = span(W4, rows, K / 2, K / 2, 1), s4r = span(S4, K / 256, rows * 8, rows * 8, 1),
              br = span(bias_cat, 1, rows, rows, 2);
  if (overlap(w4r, s4r) || overlap(w4r, br) || overlap(s4r, br)) return refuse(FRT_E_INVALID, "pack_mxfp4: outputs overlap");
  for (int i = 0; i < n_sib; ++i) {
    const Range wr = span(sibs[i].w, sibs[i].rows, K, K, 2), bb = span(sibs[i].b, 1, sibs[i].rows, sibs[i].rows, 2);
    if (overlap(wr, w4r) || overlap(wr, s4r) || overlap(wr, br) || overlap(bb, w4r) || overlap(bb, s4r) ||
        overlap(bb, br))
      return refuse(FRT_E_INVALID, "pack_mxfp4: sibling %d overlaps an output", i);
  }
  return hip_status(frt::launch_pack_mxfp4(sibs, n_sib, K, W4, S4, bias_cat, (hipStream_t)stream), "pack_mxfp4 launch");
}

int frt_ada_norm_quant_mxfp4(void* stream, int64_t M, int64_t D, const uint16_t* residual, int64_t ld_res,
                             const uint16_t* x, int64_t ld_x, const uint16_t* gate, int64_t ld_gate,
                             const uint16_t* weight, const uint16_t* mod, int64_t ld_mod, float eps,
                             uint16_t* residual_out, int64_t ld_rout, uint8_t* out_fp4, int64_t ld_out,
                             uint8_t* out_scale, int64_t ld_sc, uint16_t* gate_out, int64_t ld_gout) {
  if (M < 0) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: M=%lld < 0", (long long)M);
  if (D < kDMin || D > kDMax || D % 256)
    return refuse(FRT_E_INVALID, "ada_norm_mxfp4: D=%lld must be a multiple of 256 in [512, 16384]", (long long)D);
  if (M > (int64_t)0x7fffffff) return refuse(FRT_E_UNSUPPORTED, "ada_norm_mxfp4: M too large");
  if (residual == nullptr || mod == nullptr || out_fp4 == nullptr || out_scale == nullptr)
    return refuse(FRT_E_INVALID, "ada_norm_mxfp4: residual, mod, out_fp4 and out_scale are required");
  if (ld_res < D || (x != nullptr && ld_x < D)) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld < D");
  if (gate != nullptr && ld_gate != 0 && ld_gate < D)
    return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld_gate must be 0 (broadcast) or >= D");
  if (ld_mod != 0 && ld_mod < 3 * D) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld_mod must be 0 or >= 3*D");
  if (ld_out < D / 2 || ld_out % 4) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld_out must be >= D/2 and a multiple of 4");
  if (ld_sc < 8 * M) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld_sc (the scale run stride) < 8*M");
  if (residual_out != nullptr && ld_rout < D) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld_rout < D");
  if (gate_out != nullptr && ld_gout < D) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: ld_gout < D");
  const bool al = aligned(residual, 16) && ld_res % 8 == 0 && (x == nullptr || (aligned(x, 16) && ld_x % 8 == 0)) &&
                  (gate == nullptr || (aligned(gate, 16) && ld_gate % 8 == 0)) &&
                  (weight == nullptr || aligned(weight, 16)) && aligned(mod, 16) && ld_mod % 8 == 0 &&
                  (residual_out == nullptr || (aligned(residual_out, 16) && ld_rout % 8 == 0)) &&
                  aligned(out_fp4, 4) && (gate_out == nullptr || (aligned(gate_out, 16) && ld_gout % 8 == 0));
  if (!al) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: 16-byte aligned inputs with ld % 8 == 0 (out_fp4: 4-byte) required");
  if (M == 0) return ok();
  const int64_t mrows = ld_mod ? M : 1, grows = ld_gate ? M : 1;
  const Range in[] = {span(residual, M, D, ld_res, 2), span(x, M, D, ld_x, 2),
                      span(gate, grows, D, ld_gate ? ld_gate : D, 2), span(weight, 1, D, D, 2),
                      span(mod, mrows, 3 * D, ld_mod ? ld_mod : 3 * D, 2)};
  const Range outs[] = {span(residual_out, M, D, ld_rout, 2), span(out_fp4, M, D / 2, ld_out, 1),
                        span(out_scale, D / 256, 8 * M, ld_sc, 1), span(gate_out, M, D, ld_gout, 2)};
  const bool inplace = residual_out != nullptr && residual_out == residual && ld_rout == ld_res;
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 5; ++i) {
      if (o == 0 && i == 0 && inplace) continue;
      if (overlap(outs[o], in[i])) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: output %d overlaps input %d", o, i);
    }
    for (int p = o + 1; p < 4; ++p)
      if (overlap(outs[o], outs[p])) return refuse(FRT_E_INVALID, "ada_norm_mxfp4: outputs %d and %d overlap", o, p);
  }
  frt::AdaArgs a{residual, ld_res, x, ld_x, gate, ld_gate, weight, mod, ld_mod,
                 nullptr, eps, residual_out, ld_rout, out_fp4, ld_out, gate_out, ld_gout,
                 nullptr, 0, nullptr, M, (int)D, out_scale, ld_sc};
  if (x == nullptr || gate == nullptr) {
    a.x = nullptr;
    a.gate = nullptr;
  }
  return hip_status(frt::launch_ada_norm_mxfp4(a, (hipStream_t)stream), "ada_norm_mxfp4 launch");
}

int frt_packed_gemm_mxfp4_split(void* stream, int64_t M, int64_t K, const uint8_t* x4, int64_t ld_x4,
                                const uint8_t* xs, int64_t ld_xs, const uint8_t* W4, const uint8_t* S4,
                                int64_t N_total, const uint16_t* bias_cat, int n_split, const int64_t* split_n,
                                void* const* out, const int64_t* ld_out, int out_dtype) {
  if (M < 0) return refuse(FRT_E_INVALID, "gemm_mxfp4: M=%lld < 0", (long long)M);
  if (K < 512 || K > 16384 || K % 256)
    return refuse(FRT_E_INVALID, "gemm_mxfp4: K=%lld must be a multiple of 256 in [512, 16384]", (long long)K);
  if (xs == nullptr || S4 == nullptr) return refuse(FRT_E_INVALID, "gemm_mxfp4: xs and S4 are required");
  if (ld_xs < 8 * M || !aligned(xs, 4) || ld_xs % 4 || !aligned(S4, 4))
    return refuse(FRT_E_INVALID, "gemm_mxfp4: scales 4-byte aligned, ld_xs (run stride) >= 8*M and a multiple of 4");
  // the packed GEMM's own contract on the code bytes (K/2 per row): shapes,
  // 16-byte alignment, ld % 16, splits and output overlaps; the FP8 scale
  // pointers are not used, so the scale buffers stand in for them
  frt::GemmArgs a;
  const int rc = gemm_prepare(M, K, K / 2, x4, ld_x4, W4, N_total, reinterpret_cast<const float*>(xs),
                              reinterpret_cast<const float*>(S4), bias_cat, n_split, split_n, out, ld_out,
                              out_dtype, nullptr, 0, a);
  if (rc != FRT_OK) return rc;
  if (M == 0) return ok();
  const Range sar = span(xs, K / 256, 8 * M, ld_xs, 1), sbr = span(S4, K / 256, 8 * N_total, 8 * N_total, 1);
  for (int s = 0; s < n_split; ++s) {
    const Range o = span(out[s], M, split_n[s], ld_out[s], out_dtype ? 4 : 2);
    if (overlap(o, sar) || overlap(o, sbr)) return refuse(FRT_E_INVALID, "gemm_mxfp4: output %d overlaps a scale buffer", s);
  }
  a.K = (int)K;
  a.act_scale = nullptr;
  a.w_scale = nullptr;
  a.sa = xs;
  a.ld_sa = ld_xs;
  a.sb = S4;
  return hip_status(frt::launch_gemm_mxfp4(a, (hipStream_t)stream), "gemm_mxfp4 launch");
}

namespace {

// The MXFP4 gate/up GEMM with the GEGLU epilogue: FP8 codes at out_scale
// (out_fp8) or MXFP4 codes + block scales (out_fp4, out_sc).
int mx_geglu(const char* who, void* stream, int64_t M, int64_t K, const uint8_t* x4, int64_t ld_x4,
             const uint8_t* xs, int64_t ld_xs, const uint8_t* W4, const uint8_t* S4, int64_t H,
             const uint16_t* bias_cat, const float* out_scale, uint8_t* out_fp8, uint8_t* out_fp4, int64_t ld_out,
             uint8_t* out_sc, int64_t ld_sc) {
  const bool mxo = out_fp4 != nullptr;
  if (M < 0) return refuse(FRT_E_INVALID, "%s: M=%lld < 0", who, (long long)M);
  if (K < 512 || K > 16384 || K % 256)
    return refuse(FRT_E_INVALID, "%s: K=%lld must be a multiple of 256 in [512, 16384]", who, (long long)K);
  if (H < 1 || (mxo && H % 256))
    return refuse(FRT_E_INVALID, "%s: H=%lld must be >= 1%s", who, (long long)H, mxo ? " and a multiple of 256" : "");
  if (M > (1 << 24) || 2 * H > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "%s: M or 2H too large", who);
  if (x4 == nullptr || xs == nullptr || W4 == nullptr || S4 == nullptr ||
      (mxo ? out_sc == nullptr : (out_scale == nullptr || out_fp8 == nullptr)))
    return refuse(FRT_E_INVALID, "%s: x4, xs, W4, S4 and the outputs%s are required", who,
                  mxo ? "" : " (with out_scale)");
  const int64_t kb = K / 2;
  if (ld_x4 < kb || ld_x4 % 16) return refuse(FRT_E_INVALID, "%s: ld_x4 must be >= K/2 and a multiple of 16", who);
  if (!aligned(x4, 16) || !aligned(W4, 16)) return refuse(FRT_E_INVALID, "%s: x4 and W4 must be 16-byte aligned", who);
  if (ld_xs < 8 * M || !aligned(xs, 4) || ld_xs % 4 || !aligned(S4, 4))
    return refuse(FRT_E_INVALID, "%s: scales 4-byte aligned, ld_xs (run stride) >= 8*M and a multiple of 4", who);
  if ((M - 1) * ld_x4 + kb > (int64_t)0x7fffffff || 2 * H * kb > (int64_t)0x7fffffff)
    return refuse(FRT_E_UNSUPPORTED, "%s: operand larger than 2 GiB", who);
  if (mxo && (ld_out < H / 2 || ld_out % 4 || !aligned(out_fp4, 4) || ld_sc < 8 * M))
    return refuse(FRT_E_INVALID, "%s: out_fp4 4-byte aligned, ld_out >= H/2 and a multiple of 4, ld_sc >= 8*M", who);
  if (!mxo && ld_out < H) return refuse(FRT_E_INVALID, "%s: ld_out < H", who);
  if (M == 0) return ok();
  const Range in[] = {span(x4, M, kb, ld_x4, 1),           span(W4, 2 * H, kb, kb, 1),
                      span(bias_cat, 1, 2 * H, 2 * H, 2),  span(out_scale, 1, 1, 1, 4),
                      span(xs, K / 256, 8 * M, ld_xs, 1),  span(S4, K / 256, 16 * H, 16 * H, 1)};
  const Range o = mxo ? span(out_fp4, M, H / 2, ld_out, 1) : span(out_fp8, M, H, ld_out, 1);
  const Range so = span(out_sc, H / 256, 8 * M, ld_sc, 1);
  for (int i = 0; i < 6; ++i)
    if (overlap(o, in[i]) || overlap(so, in[i])) return refuse(FRT_E_INVALID, "%s: an output overlaps input %d", who, i);
  if (overlap(o, so)) return refuse(FRT_E_INVALID, "%s: the codes overlap the scales", who);
  frt::GemmArgs a{};
  a.x = x4;
  a.ld_x = ld_x4;
  a.w = W4;
  a.bias = bias_cat;
  a.M = (int)M;
  a.N = (int)(2 * H);
  a.K = (int)K;
  a.H = (int)H;
  if (mxo) {
    a.q4 = out_fp4;
    a.ld_q4 = ld_out;
    a.sc4 = out_sc;
    a.ld_sc4 = ld_sc;
  } else {
    a.q8 = out_fp8;
    a.ld_q8 = ld_out;
    a.q_scale = out_scale;
  }
  a.sa = xs;
  a.ld_sa = ld_xs;
  a.sb = S4;
  return hip_status(frt::launch_gemm_mxfp4_geglu(a, (hipStream_t)stream), who);
}

}  // namespace

int frt_packed_gemm_mxfp4_geglu_quant(void* stream, int64_t M, int64_t K, const uint8_t* x4, int64_t ld_x4,
                                      const uint8_t* xs, int64_t ld_xs, const uint8_t* W4, const uint8_t* S4,
                                      int64_t H, const uint16_t* bias_cat, const float* out_scale, uint8_t* out_fp8,
                                      int64_t ld_out) {
  return mx_geglu("gemm_mxfp4_geglu", stream, M, K, x4, ld_x4, xs, ld_xs, W4, S4, H, bias_cat, out_scale, out_fp8,
                  nullptr, ld_out, nullptr, 0);
}

int frt_packed_gemm_mxfp4_geglu_mxfp4(void* stream, int64_t M, int64_t K, const uint8_t* x4, int64_t ld_x4,
                                      const uint8_t* xs, int64_t ld_xs, const uint8_t* W4, const uint8_t* S4,
                                      int64_t H, const uint16_t* bias_cat, uint8_t* out_fp4, int64_t ld_out,
                                      uint8_t* out_scale, int64_t ld_sc) {
  if (out_fp4 == nullptr) return refuse(FRT_E_INVALID, "gemm_mxfp4_geglu_mxfp4: out_fp4 is required");
  return mx_geglu("gemm_mxfp4_geglu_mxfp4", stream, M, K, x4, ld_x4, xs, ld_xs, W4, S4, H, bias_cat, nullptr, nullptr,
                  out_fp4, ld_out, out_scale, ld_sc);
}

int frt_interleave_pairs_bf16(void* stream, int nheads, int hd, int64_t K, const uint16_t* src, uint16_t* dst) {
  if (nheads < 1 || hd < 2 || hd % 2) return refuse(FRT_E_INVALID, "interleave: nheads >= 1 and an even hd >= 2");
  if (K < 1) return refuse(FRT_E_INVALID, "interleave: K < 1");
  if ((int64_t)nheads * hd > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "interleave: too many rows");
  if (src == nullptr || dst == nullptr) return refuse(FRT_E_INVALID, "interleave: src and dst are required");
  if (!aligned(src, 2) || !aligned(dst, 2)) return refuse(FRT_E_INVALID, "interleave: src/dst misaligned");
  const int64_t rows = (int64_t)nheads * hd;
  if (overlap(span(src, rows, K, K, 2), span(dst, rows, K, K, 2)))
    return refuse(FRT_E_INVALID, "interleave: dst overlaps src");
  const int vec = (K % 8 == 0 && aligned(src, 16) && aligned(dst, 16)) ? 8 : 1;
  return hip_status(frt::launch_interleave(src, dst, nheads, hd, K, vec, (hipStream_t)stream), "interleave launch");
}

namespace {

// Shared contract of the split + RoPE + KV-cache outputs.
int check_rope_outputs(const char* who, int64_t S, int nh, int kv, int hd, const uint16_t* rope, int64_t P,
                       int64_t T, const uint16_t* q_out, const uint16_t* k_cache, const uint16_t* v_cache,
                       const Range* inputs, int n_in) {
  if (S < 0) return refuse(FRT_E_INVALID, "%s: S=%lld < 0", who, (long long)S);
  if (nh < 1 || kv < 1 || hd < 2 || hd % 2)
    return refuse(FRT_E_INVALID, "%s: nh >= 1, kv >= 1 and an even hd >= 2 are required", who);
  if ((int64_t)(nh + 2 * kv) * hd > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "%s: too many columns", who);
  if (P < 0 || T < 1 || P + S > T)
    return refuse(FRT_E_INVALID, "%s: cache rows P .. P+S-1 must lie in [0, T)", who);
  if (rope == nullptr || q_out == nullptr || k_cache == nullptr || v_cache == nullptr)
    return refuse(FRT_E_INVALID, "%s: rope, q_out, k_cache and v_cache are required", who);
  if (!aligned(rope, 4) || !aligned(q_out, 2) || !aligned(k_cache, 2) || !aligned(v_cache, 2))
    return refuse(FRT_E_INVALID, "%s: rope must be 4-byte and the outputs 2-byte aligned", who);
  if (S == 0) return FRT_OK;
  const int64_t nk = (int64_t)kv * hd;
  const Range outs[3] = {span(q_out, S, (int64_t)nh * hd, (int64_t)nh * hd, 2),
                         span(k_cache + P * nk, S, nk, nk, 2), span(v_cache + P * nk, S, nk, nk, 2)};
  const Range rr = span(rope, S, hd, hd, 2);
  for (int o = 0; o < 3; ++o) {
    if (overlap(outs[o], rr)) return refuse(FRT_E_INVALID, "%s: output %d overlaps rope", who, o);
    for (int i = 0; i < n_in; ++i)
      if (overlap(outs[o], inputs[i])) return refuse(FRT_E_INVALID, "%s: output %d overlaps input %d", who, o, i);
    for (int q = o + 1; q < 3; ++q)
      if (overlap(outs[o], outs[q])) return refuse(FRT_E_INVALID, "%s: outputs %d and %d overlap", who, o, q);
  }
  return FRT_OK;
}

}  // namespace

int frt_qkv_split_rope_kvcache(void* stream, int64_t S, int nh, int kv, int hd, const uint16_t* qkv,
                               int64_t ld_qkv, const uint16_t* rope, int64_t P, int64_t T, uint16_t* q_out,
                               uint16_t* k_cache, uint16_t* v_cache) {
  const int64_t ncol = (int64_t)(nh + 2 * kv) * hd;
  if (qkv == nullptr) return refuse(FRT_E_INVALID, "rope_split: qkv is required");
  if (nh >= 1 && kv >= 1 && ld_qkv < ncol) return refuse(FRT_E_INVALID, "rope_split: ld_qkv < (nh + 2kv) hd");
  if (!aligned(qkv, 4) || ld_qkv % 2)
    return refuse(FRT_E_INVALID, "rope_split: qkv must be 4-byte aligned with an even ld_qkv");
  const Range in[1] = {span(qkv, S, ncol, ld_qkv, 2)};
  const int rc = check_rope_outputs("rope_split", S, nh, kv, hd, rope, P, T, q_out, k_cache, v_cache, in, 1);
  if (rc != FRT_OK) return rc;
  if (S == 0) return ok();
  const bool vec8 = hd % 8 == 0 && ld_qkv % 8 == 0 && aligned(qkv, 16) && aligned(rope, 16) && aligned(q_out, 16) &&
                    aligned(k_cache, 16) && aligned(v_cache, 16);
  frt::RopeArgs a{qkv, ld_qkv, rope, nh, kv, hd, S, P, q_out, k_cache, v_cache};
  return hip_status(frt::launch_rope_split(a, vec8 ? 8 : 2, (hipStream_t)stream), "rope_split launch");
}

int frt_packed_gemm_fp8_qkv_rope(void* stream, int64_t M, int64_t K, const uint8_t* x8, int64_t ld_x,
                                 const uint8_t* W8, int nh, int kv, int hd, const float* act_scale,
                                 const float* w_scale, const uint16_t* bias_cat, const uint16_t* rope, int64_t P,
                                 int64_t T, uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache) {
  if (M < 0) return refuse(FRT_E_INVALID, "gemm_rope: M=%lld < 0", (long long)M);
  if (K < 512 || K > 16384) return refuse(FRT_E_INVALID, "gemm_rope: K=%lld outside [512, 16384]", (long long)K);
  if (K % 16) return refuse(FRT_E_UNSUPPORTED, "gemm_rope: K=%lld not a multiple of 16", (long long)K);
  if (M > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "gemm_rope: M too large");
  if (x8 == nullptr || W8 == nullptr || act_scale == nullptr || w_scale == nullptr)
    return refuse(FRT_E_INVALID, "gemm_rope: x8, W8, act_scale and w_scale are required");
  if (ld_x < K || ld_x % 16) return refuse(FRT_E_INVALID, "gemm_rope: ld_x must be >= K and a multiple of 16");
  if (!aligned(x8, 16) || !aligned(W8, 16)) return refuse(FRT_E_INVALID, "gemm_rope: x8 and W8 must be 16-byte aligned");
  const int64_t N = (nh >= 1 && kv >= 1 && hd >= 2) ? (int64_t)(nh + 2 * kv) * hd : 0;
  if ((M - 1) * ld_x + K > (int64_t)0x7fffffff || N * K > (int64_t)0x7fffffff)
    return refuse(FRT_E_UNSUPPORTED, "gemm_rope: operand larger than 2 GiB");
  const Range in[5] = {span(x8, M, K, ld_x, 1), span(W8, N, K, K, 1), span(bias_cat, 1, N, N, 2),
                       span(act_scale, 1, 1, 1, 4), span(w_scale, 1, 1, 1, 4)};
  const int rc = check_rope_outputs("gemm_rope", M, nh, kv, hd, rope, P, T, q_out, k_cache, v_cache, in, 5);
  if (rc != FRT_OK) return rc;
  if (M == 0) return ok();
  frt::GemmArgs a{};
  a.x = x8;
  a.ld_x = ld_x;
  a.w = W8;
  a.act_scale = act_scale;
  a.w_scale = w_scale;
  a.bias = bias_cat;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.rope = rope;
  a.nh = nh;
  a.kv = kv;
  a.hd = hd;
  a.P = P;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return hip_status(frt::launch_gemm_rope(a, (hipStream_t)stream), "gemm_rope launch");
}

int frt_packed_gemm_mxfp4_qkv_rope(void* stream, int64_t M, int64_t K, const uint8_t* x4, int64_t ld_x4,
                                   const uint8_t* xs, int64_t ld_xs, const uint8_t* W4, const uint8_t* S4, int nh,
                                   int kv, int hd, const uint16_t* bias_cat, const uint16_t* rope, int64_t P,
                                   int64_t T, uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache) {
  if (M < 0) return refuse(FRT_E_INVALID, "gemm_mxfp4_rope: M=%lld < 0", (long long)M);
  if (K < 512 || K > 16384 || K % 256)
    return refuse(FRT_E_INVALID, "gemm_mxfp4_rope: K=%lld must be a multiple of 256 in [512, 16384]", (long long)K);
  if (M > (1 << 24)) return refuse(FRT_E_UNSUPPORTED, "gemm_mxfp4_rope: M too large");
  if (x4 == nullptr || xs == nullptr || W4 == nullptr || S4 == nullptr)
    return refuse(FRT_E_INVALID, "gemm_mxfp4_rope: x4, xs, W4 and S4 are required");
  const int64_t kb = K / 2;
  if (ld_x4 < kb || ld_x4 % 16)
    return refuse(FRT_E_INVALID, "gemm_mxfp4_rope: ld_x4 must be >= K/2 and a multiple of 16");
  if (!aligned(x4, 16) || !aligned(W4, 16))
    return refuse(FRT_E_INVALID, "gemm_mxfp4_rope: x4 and W4 must be 16-byte aligned");
  if (ld_xs < 8 * M || !aligned(xs, 4) || ld_xs % 4 || !aligned(S4, 4))
    return refuse(FRT_E_INVALID,
                  "gemm_mxfp4_rope: scales 4-byte aligned, ld_xs (run stride) >= 8*M and a multiple of 4");
  const int64_t N = (nh >= 1 && kv >= 1 && hd >= 2) ? (int64_t)(nh + 2 * kv) * hd : 0;
  if ((M - 1) * ld_x4 + kb > (int64_t)0x7fffffff || N * kb > (int64_t)0x7fffffff)
    return refuse(FRT_E_UNSUPPORTED, "gemm_mxfp4_rope: operand larger than 2 GiB");
  const Range in[5] = {span(x4, M, kb, ld_x4, 1), span(W4, N, kb, kb, 1), span(bias_cat, 1, N, N, 2),
                       span(xs, K / 256, 8 * M, ld_xs, 1), span(S4, K / 256, 8 * N, 8 * N, 1)};
  const int rc = check_rope_outputs("gemm_mxfp4_rope", M, nh, kv, hd, rope, P, T, q_out, k_cache, v_cache, in, 5);
  if (rc != FRT_OK) return rc;
  if (M == 0) return ok();
  frt::GemmArgs a{};
  a.x = x4;
  a.ld_x = ld_x4;
  a.w = W4;
  a.bias = bias_cat;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.sa = xs;
  a.ld_sa = ld_xs;
  a.sb = S4;
  a.rope = rope;
  a.nh = nh;
  a.kv = kv;
  a.hd = hd;
  a.P = P;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return hip_status(frt::launch_gemm_mxfp4_rope(a, (hipStream_t)stream), "gemm_mxfp4_rope launch");
}

}  // extern "C"
