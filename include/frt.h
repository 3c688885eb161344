/*
 * frt.h — C ABI of the MI355X (gfx950) FP8 norm-quantize producers and the
 * packed sibling-projection FP8 GEMM.
 *
 * The operations follow the flashrt-structures 0.2.0 wheel pages:
 *   - impls/adarms_stack/fp8_chain.py: the fused gated-residual AdaRMS
 *     producer that feeds the merged QKV and gate/up GEMMs, and the stack's
 *     fp32 tail that prints its arithmetic;
 *   - impls/modnorm_qkv_chain/fp8_ptok_table.py: the per-token-table
 *     no-affine adaptive LayerNorm producer;
 *   - impls/qkv_pack/fp8_static.py: `_pack_weights` (one joint per-tensor
 *     scale over the concatenated siblings) and `PackedLinear._run` (the
 *     packed FP8 GEMM with optional bias whose columns are handed out per
 *     sibling);
 *   - fp8_chain.py's FFN tail: the merged gate/up output turned into the
 *     FP8 input of the down projection by a tanh-GELU GEGLU quantiser,
 *     standalone or as the gate/up GEMM's epilogue;
 *   - fp8_chain.py's attention head: the merged QKV output split, rotated
 *     by adjacent-pair RoPE and written to q and the KV caches, standalone
 *     or as the QKV GEMM's epilogue;
 *   - projections without a producer: the static quantiser of a bf16
 *     tensor and the bf16-input form of the packed GEMM;
 *   - an MXFP4 band (producer, weight pack, GEMM) in the place of the
 *     pages' NVFP4 band.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers unless marked [host].
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *     asynchronous and stream-ordered; no call synchronises the host.
 *   - The caller owns every buffer. No call allocates or frees memory, and
 *     the library keeps no state between calls (except the thread-local
 *     error string).
 *   - bf16 tensors are passed as uint16_t bit patterns, FP8 as uint8_t
 *     e4m3fn codes (OCP FP8: bias 7, max 448, 0x7F/0xFF NaN, no infinity).
 *   - Leading dimensions (`ld_*`) are in ELEMENTS of the tensor's own type.
 *   - Row counts are logical: any M not above the caller's buffer rows is
 *     legal and only M rows are read or written (the pages' row *capacity*
 *     contract). M = 0 is a no-op returning FRT_OK.
 *   - Device-resident scalars (act_scale, w_scale) are never read on the
 *     host.
 *   - Return value: FRT_OK, or a negative status with a reason available
 *     from frt_last_error() ("refused: ..."). FRT_E_INVALID = a violated
 *     contract (bad pointer, size, stride, alignment or aliasing);
 *     FRT_E_UNSUPPORTED = legal but outside what the kernels implement;
 *     FRT_E_HIP = a HIP launch error. Validation happens before any launch,
 *     so a refused call has not touched any buffer.
 */
#ifndef FRT_H_
#define FRT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FRT_OK 0
#define FRT_E_INVALID (-1)
#define FRT_E_UNSUPPORTED (-2)
#define FRT_E_HIP (-3)

/* Largest number of column splits (siblings) one packed call can serve. */
#define FRT_MAX_SPLITS 16

/* Reason for the last non-OK status on this thread ("" if none). */
const char* frt_last_error(void);

/* ABI version of this header (bumped on any signature change). */
int frt_abi_version(void);

/*
 * frt_ada_norm_quant_fp8 — gated residual + AdaRMS + static per-tensor FP8.
 *
 * Source: fp8_chain.py, `_band_elements` (the producer call with the
 * residual, the delta x, the previous site's gate, a ones norm weight, one
 * style row, the site's activation scale, eps, `out=` FP8 and `gate_out=`)
 * and `_make_run` / the stack tail for the arithmetic. Per row m < M and
 * column d < D:
 *   h        = fl32(residual[m,d] + gate[m,d] * x[m,d])     (single rounding)
 *   residual_out[m,d] = bf16_rne(h)
 *   r_m      = 1 / sqrt(sum_d h^2 / D + eps)
 *   y        = (h * r_m * weight[d]) * (1 + scale[d]) + shift[d]
 *   out_fp8  = e4m3_rne(clamp(fl32(y / act_scale), -448, 448))
 *   gate_out[m,d] = gate_chunk[d]
 * where the modulation row is mod[m', 0:D] = scale, mod[m', D:2D] = shift,
 * mod[m', 2D:3D] = gate_chunk (m' = m, or 0 when ld_mod = 0). y is kept in
 * fp32 and is not rounded to bf16 before the quantiser.
 *
 *   M, D          rows; hidden size. D in [512, 16384], even.
 *   residual      bf16 [M, ld_res]. Required.
 *   x             bf16 [M, ld_x] delta; NULL => h = residual.
 *   gate          bf16 previous-site gate; ld_gate = 0 => one row [D]
 *                 broadcast to every row, else [M, ld_gate]. NULL => zero
 *                 gate (h = residual, layer 0 of a chain).
 *   weight        bf16 [D] norm weight; NULL => ones.
 *   mod           bf16 [*, ld_mod] rows of 3D = [scale | shift | gate];
 *                 ld_mod = 0 => one row broadcast. Required.
 *   act_scale     fp32 [1] static scale (> 0). Required iff out_fp8.
 *   eps           added to the mean square.
 *   residual_out  bf16 [M, ld_rout]; may be exactly `residual` with the same
 *                 ld (in-place update). Any other overlap with an input is
 *                 refused. NULL => not written.
 *   out_fp8       e4m3fn [M, ld_out]; NULL => not written.
 *   gate_out      bf16 [M, ld_gout]; NULL => not written.
 *   y_f32         fp32 [M, ld_y] pre-quantisation y (diagnostic); NULL =>
 *                 not written.
 *   amax_out      fp32 [1]: atomically raised to max |y| over the call
 *                 (calibration); the caller initialises it. NULL => off.
 * Alignment: every pointer 16-byte aligned and every ld a multiple of 8
 * (16 for out_fp8) with D % 8 == 0 takes the vector path; otherwise 4-byte
 * alignment is required (FRT_E_INVALID if not).
 */
int frt_ada_norm_quant_fp8(void* stream, int64_t M, int64_t D,
                           const uint16_t* residual, int64_t ld_res,
                           const uint16_t* x, int64_t ld_x,
                           const uint16_t* gate, int64_t ld_gate,
                           const uint16_t* weight,
                           const uint16_t* mod, int64_t ld_mod,
                           const float* act_scale, float eps,
                           uint16_t* residual_out, int64_t ld_rout,
                           uint8_t* out_fp8, int64_t ld_out,
                           uint16_t* gate_out, int64_t ld_gout,
                           float* y_f32, int64_t ld_y,
                           float* amax_out);

/*
 * frt_ptok_table_norm_quant_fp8 — per-token-table no-affine adaptive
 * LayerNorm + static per-tensor FP8.
 *
 * Source: fp8_ptok_table.py, module docstring (table add + chunk selection
 * + no-affine LayerNorm + modulation + static FP8 quantize in one pass,
 * never materialising the six chunks), `PerTokenModChainBlock.forward` (the
 * producer call with x2d, the bf16 temb, the fp32 table, the site scale,
 * the shift and scale chunk indices, eps), `_ATTN_CHUNKS` / `_FFN_CHUNKS`
 * (chunk roles shift, scale, gate) and `SUPPORT` (6 chunks, D in
 * [512, 16384], even). Per row r < R, column d < D:
 *   shift = fl32(table[shift_idx, d] + temb[r, shift_idx, d])
 *   scale = fl32(table[scale_idx, d] + temb[r, scale_idx, d])
 *   mu    = mean_d x[r, d];  var = mean_d (x[r, d] - mu)^2   (biased)
 *   y     = (x - mu) / sqrt(var + eps) * (1 + scale) + shift
 *   out_fp8 = e4m3_rne(clamp(fl32(y / act_scale), -448, 448))
 *
 *   R, D          rows (= B*M tokens); hidden size. D in [512, 16384], even.
 *   C             chunks per temb row; must be 6.
 *   x             bf16 [R, ld_x].
 *   temb          bf16 [R, C, D] with row stride ld_temb (>= C*D) elements;
 *                 row r pairs with x row r. Only the two selected chunks
 *                 are read.
 *   table         fp32 [C, D] contiguous.
 *   act_scale     fp32 [1] (> 0). Required iff out_fp8.
 *   shift_idx, scale_idx   chunk indices in [0, C).
 *   out_fp8, y_f32, amax_out   as in frt_ada_norm_quant_fp8.
 * Alignment as in frt_ada_norm_quant_fp8 (table 16-byte aligned for the
 * vector path).
 */
int frt_ptok_table_norm_quant_fp8(void* stream, int64_t R, int64_t D, int C,
                                  const uint16_t* x, int64_t ld_x,
                                  const uint16_t* temb, int64_t ld_temb,
                                  const float* table,
                                  const float* act_scale,
                                  int shift_idx, int scale_idx, float eps,
                                  uint8_t* out_fp8, int64_t ld_out,
                                  float* y_f32, int64_t ld_y,
                                  float* amax_out);

/*
 * frt_pack_weights_fp8 — pack sibling projections into one FP8 matrix with
 * one joint per-tensor scale.
 *
 * Source: qkv_pack/fp8_static.py `_pack_weights` (also `_q8` in
 * fp8_ptok_table.py). With W = concat_i W_i along the output axis:
 *   w_scale = max(fl32(max|W| / 448), 1e-8)
 *   W8      = e4m3_rne(clamp(fl32(W / w_scale), -448, 448))  (true division)
 *   bias_cat = concat_i (b_i, or zeros for a sibling without bias)
 * The result is bit-exact to that definition.
 *
 *   n_sib         number of siblings, 1 .. FRT_MAX_SPLITS.
 *   N_i   [host]  int64 [n_sib] output widths (each >= 1).
 *   K             shared input width, >= 1.
 *   W_i   [host]  array of n_sib device pointers to bf16 [N_i, K]
 *                 (checkpoint layout, K contiguous, rows packed).
 *   b_i   [host]  array of n_sib device pointers to bf16 [N_i] or NULL
 *                 entries; the array itself NULL => no biases.
 *   W8            e4m3fn [sum N_i, K] output, rows packed.
 *   w_scale       fp32 [1] output. Used as the amax accumulator while the
 *                 call runs; holds the scale when the stream reaches the
 *                 call's end.
 *   bias_cat      bf16 [sum N_i] output, or NULL => not written.
 * Non-finite weights make w_scale and the codes NaN, as the definition does.
 */
int frt_pack_weights_fp8(void* stream, int n_sib, const int64_t* N_i,
                         int64_t K, const uint16_t* const* W_i,
                         const uint16_t* const* b_i, uint8_t* W8,
                         float* w_scale, uint16_t* bias_cat);

/*
 * Workspace bytes frt_packed_gemm_fp8_split needs for this shape on the
 * current device. The present tile plans need none, so this returns 0 for
 * every shape; callers that query it and pass a workspace of at least this
 * size stay correct if a later plan needs one (such a workspace would have
 * to be zero-filled once before first use and be left zero-filled by every
 * call; calls sharing one must not overlap).
 */
size_t frt_packed_gemm_fp8_workspace_size(int64_t M, int64_t N_total,
                                          int64_t K);

/*
 * frt_packed_gemm_fp8_split — packed FP8 GEMM with dequant, bias and
 * column-split epilogue.
 *
 * Source: qkv_pack/fp8_static.py `PackedLinear._run` (fp8_gemm_bf16 /
 * fp8_linear_bias_bf16 with act_scale and w_scale into the [M, sum N_i]
 * output; sibling i takes columns [off_i, off_i + N_i)) and fp8_chain.py
 * `_quantize` (alpha = act_scale * w_scale folded into one factor). For
 * m < M, n < N_total:
 *   acc[m, n] = sum_k dec(x8[m, k]) * dec(W8[n, k])      (fp32 accumulate)
 *   v         = fl32(alpha * acc[m, n]) + bias_cat[n],  alpha = fl32(as*ws)
 *   out_s[m, n - off_s] = bf16_rne(v)   (or v itself for out_dtype 1)
 * with s the split holding column n (off_s = split_n[0] + ... + split_n[s-1]).
 * The bias is added once, before the single output rounding.
 *
 *   M             rows (logical; 0 => no-op).
 *   K             reduction size: 512 <= K <= 16384 and K % 16 == 0.
 *   x8            e4m3fn [M, ld_x] (K contiguous); ld_x >= K, ld_x % 16 == 0,
 *                 16-byte aligned.
 *   W8            e4m3fn [N_total, K] packed rows (ld = K), 16-byte aligned.
 *   act_scale, w_scale   fp32 [1] each.
 *   bias_cat      bf16 [N_total] or NULL (no bias).
 *   n_split       1 .. FRT_MAX_SPLITS.
 *   split_n [host] int64 [n_split], each >= 1, summing to N_total.
 *   out     [host] n_split device pointers; split s is [M, split_n[s]] with
 *                 row stride ld_out[s] >= split_n[s] (elements). One pointer
 *                 may cover several adjacent columns runs by merging them
 *                 into one split. Output regions must not overlap each
 *                 other or the inputs. 4-byte aligned (bf16: ld even).
 *   ld_out  [host] int64 [n_split].
 *   out_dtype     0 = bf16, 1 = fp32 (parity / diagnostics).
 *   workspace, ws_bytes   at least frt_packed_gemm_fp8_workspace_size
 *                 bytes (NULL/0 allowed when that is 0, as it is for every
 *                 shape today); a smaller one is refused before any launch.
 *
 * Layout and speed: with bf16 outputs whose split widths and row strides are
 * multiples of 8 elements and whose pointers are 16-byte aligned, the
 * large-M plan (256 x 256 tiles) stores whole 128-byte row segments; any
 * other accepted layout gives the same bits through per-element stores.
 */
int frt_packed_gemm_fp8_split(void* stream, int64_t M, int64_t K,
                              const uint8_t* x8, int64_t ld_x,
                              const uint8_t* W8, int64_t N_total,
                              const float* act_scale, const float* w_scale,
                              const uint16_t* bias_cat, int n_split,
                              const int64_t* split_n, void* const* out,
                              const int64_t* ld_out, int out_dtype,
                              void* workspace, size_t ws_bytes);

/*
 * frt_geglu_quant_fp8 — GEGLU of a merged gate/up row + static per-tensor
 * FP8 (the FFN's down-projection input).
 *
 * Source: fp8_chain.py, `_quantize` (gate and up packed as one matrix, gate
 * rows first, so a merged output row is [gate | up]) and `_band_elements`
 * (`down_project`: the merged GEGLU + static FP8 quantiser feeding the
 * down projection); the chain's bind admits only tanh-GELU FFNs. For
 * m < M, j < H:
 *   y   = gelu_tanh(gu[m, j]) * gu[m, H + j]                       (fp32)
 *         gelu_tanh(v) = 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
 *   out_fp8[m, j] = e4m3_rne(clamp(fl32(y / act_scale), -448, 448))
 *
 *   M, H          rows; width of each half (1 <= H <= 2^24).
 *   gu            bf16 [M, ld_gu], ld_gu >= 2H: gate in [0, H), up in
 *                 [H, 2H).
 *   act_scale     fp32 [1] (> 0). Required iff out_fp8.
 *   out_fp8       e4m3fn [M, ld_out]; NULL => not written.
 *   y_f32         fp32 [M, ld_y] pre-quantisation y (diagnostic); NULL =>
 *                 not written.
 *   amax_out      fp32 [1]: atomically raised to max |y| (calibration of
 *                 the down projection's scale); the caller initialises it.
 * At least one output. Outputs must not overlap each other or the inputs.
 * H % 8 == 0 with gu 16-byte aligned, ld_gu % 8 == 0, out_fp8 8-byte
 * aligned with ld_out % 8 == 0 and y_f32 16-byte aligned with ld_y % 4 == 0
 * takes the vector path; any other layout runs one element per thread
 * (gu 2-byte, y_f32 4-byte alignment required).
 */
int frt_geglu_quant_fp8(void* stream, int64_t M, int64_t H,
                        const uint16_t* gu, int64_t ld_gu,
                        const float* act_scale,
                        uint8_t* out_fp8, int64_t ld_out,
                        float* y_f32, int64_t ld_y, float* amax_out);

/*
 * frt_packed_gemm_fp8_geglu_quant — the merged gate/up FP8 GEMM with the
 * GEGLU quantiser as its epilogue: the [M, 2H] bf16 gate/up output never
 * reaches memory.
 *
 * Source: as frt_packed_gemm_fp8_split for the GEMM (one packed matrix,
 * alpha = act_scale * w_scale, optional bias) followed by
 * frt_geglu_quant_fp8 (fp8_chain.py `_band_elements`, `down_project`).
 * For m < M, j < H, with acc as in frt_packed_gemm_fp8_split over W8 rows
 * j (gate) and H + j (up):
 *   g = bf16_rne(fl32(alpha * acc[m, j])     + bias_cat[j])
 *   u = bf16_rne(fl32(alpha * acc[m, H + j]) + bias_cat[H + j])
 *   out_fp8[m, j] = e4m3_rne(clamp(fl32(gelu_tanh(g) * u / out_scale), +-448))
 * i.e. exactly frt_packed_gemm_fp8_split (bf16 out) followed by
 * frt_geglu_quant_fp8 on its output.
 *
 *   M, K, x8, ld_x, act_scale, w_scale   as in frt_packed_gemm_fp8_split.
 *   W8            e4m3fn [2H, K]: the H gate rows, then the H up rows (the
 *                 frt_pack_weights_fp8 result for siblings {gate, up}).
 *   H             hidden width; 2H <= 2^24.
 *   bias_cat      bf16 [2H] or NULL.
 *   out_scale     fp32 [1] static scale of the GEGLU output (> 0).
 *   out_fp8       e4m3fn [M, ld_out], ld_out >= H; must not overlap an
 *                 input.
 */
int frt_packed_gemm_fp8_geglu_quant(void* stream, int64_t M, int64_t K,
                                    const uint8_t* x8, int64_t ld_x,
                                    const uint8_t* W8, int64_t H,
                                    const float* act_scale,
                                    const float* w_scale,
                                    const uint16_t* bias_cat,
                                    const float* out_scale,
                                    uint8_t* out_fp8, int64_t ld_out);

/*
 * frt_quantize_fp8_static — static per-tensor FP8 of a bf16 tensor (the
 * producers' quantiser without a norm).
 *
 * Source: fp8_chain.py `_band_elements` (`out_project`: the attention
 * output quantised by `quantize_fp8_static_bf16` before the O projection's
 * FP8 GEMM) and impls/linear_proj/fp8_static.py (the quantize that
 * precedes the FP8 GEMM when the projection's input arrives in bf16).
 * For m < M, j < D:
 *   out_fp8[m, j] = e4m3_rne(clamp(fl32(x[m, j] / act_scale), -448, 448))
 * (x is exact in fp32; the division is correctly rounded, so the codes are
 * bit-exact to the definition).
 *
 *   M, D          rows; row width (1 <= D <= 2^24).
 *   x             bf16 [M, ld_x].
 *   act_scale     fp32 [1] (> 0). Required iff out_fp8.
 *   out_fp8       e4m3fn [M, ld_out]; NULL => not written.
 *   amax_out      fp32 [1] raised to max |x| (calibration); NULL => off.
 * At least one output; outputs must not overlap x. D % 8 == 0 with x
 * 16-byte aligned, ld_x % 8 == 0 and out_fp8 8-byte aligned with
 * ld_out % 8 == 0 takes the vector path.
 */
int frt_quantize_fp8_static(void* stream, int64_t M, int64_t D,
                            const uint16_t* x, int64_t ld_x,
                            const float* act_scale,
                            uint8_t* out_fp8, int64_t ld_out,
                            float* amax_out);

/*
 * frt_packed_gemm_bf16in_split — the packed FP8 GEMM for a projection whose
 * input arrives in bf16: the input is quantised with the static scale into
 * the caller's FP8 buffer x8, then the GEMM runs on it.
 *
 * Source: qkv_pack/fp8_static.py `PackedLinear._run` (the non-FP8 input
 * form: `bf16_fp8_linear_bias_bf16(flat, w8, bias_cat, act_scale, w_scale,
 * input_fp8=x8_buf, out=...)`) and impls/linear_proj/fp8_static.py (the
 * fused-quantize form). Exactly frt_quantize_fp8_static(x -> x8) followed
 * by frt_packed_gemm_fp8_split(x8, ...): two launches, the bias added in
 * the GEMM's epilogue.
 *
 *   x             bf16 [M, ld_x], ld_x >= K.
 *   x8            e4m3fn [M, ld_x8] written with the codes of x (the
 *                 contract of frt_packed_gemm_fp8_split's x8: 16-byte
 *                 aligned, ld_x8 >= K and a multiple of 16); must not
 *                 overlap x, the weights, scales, bias or outputs.
 *   all other arguments as in frt_packed_gemm_fp8_split.
 * Every check runs before the first launch.
 */
int frt_packed_gemm_bf16in_split(void* stream, int64_t M, int64_t K,
                                 const uint16_t* x, int64_t ld_x,
                                 uint8_t* x8, int64_t ld_x8,
                                 const uint8_t* W8, int64_t N_total,
                                 const float* act_scale, const float* w_scale,
                                 const uint16_t* bias_cat, int n_split,
                                 const int64_t* split_n, void* const* out,
                                 const int64_t* ld_out, int out_dtype,
                                 void* workspace, size_t ws_bytes);

/*
 * MXFP4 band — the MI355X counterpart of the pages' NVFP4 band (fp8_chain.py
 * `BANDS`, the `fp4` row: the norm-fed projections in 4-bit with dynamic
 * block scales, the down projection kept in static FP8). The format is OCP
 * MX FP4, which the gfx950 matrix cores take natively:
 *   - e2m1 codes (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign), two
 *     per byte, the lower-indexed element in the low nibble;
 *   - one E8M0 scale byte (2^(s-127), 0xFF = NaN) per 32 consecutive
 *     elements along the reduction axis (rows of activations, rows of
 *     [N, K] weights);
 *   - conversion by the OCP rule: scale = 2^(floor(log2(max|v|)) - 2) of the
 *     fp32 block values (byte 0 for a zero or subnormal maximum, 0xFF for
 *     NaN or inf), code = e2m1 round-to-nearest-even of v / scale,
 *     saturating at 6;
 *   - scale layout: run-major [K/256][rows][8]: the 8 block scales of each
 *     run of 256 elements of a row sit together, ordered blocks 0, 2, 4, 6,
 *     1, 3, 5, 7, and the runs of all rows for one K range are contiguous
 *     (rows 8 bytes apart, runs `ld` bytes apart), so the GEMM reads a
 *     32-row block's scales for a K range as 256 contiguous bytes.
 */

/*
 * frt_pack_weights_mxfp4 — MXFP4 pack of sibling projections (per-block
 * scales, so no joint per-tensor scale is needed).
 *
 *   n_sib, N_i [host], W_i [host], b_i [host]   as in frt_pack_weights_fp8;
 *                 every W_i 16-byte aligned.
 *   K             multiple of 256 in [512, 16384].
 *   W4            [sum N_i, K/2] code bytes (4-byte aligned).
 *   S4            scale bytes, [K/256][sum N_i][8] (run stride 8 * sum N_i).
 *   bias_cat      bf16 [sum N_i] or NULL.
 */
int frt_pack_weights_mxfp4(void* stream, int n_sib, const int64_t* N_i,
                           int64_t K, const uint16_t* const* W_i,
                           const uint16_t* const* b_i, uint8_t* W4,
                           uint8_t* S4, uint16_t* bias_cat);

/*
 * frt_ada_norm_quant_mxfp4 — the gated-residual AdaRMS producer with an
 * MXFP4 output (the FP4 twin of frt_ada_norm_quant_fp8; the pages'
 * `gate_res_ada_rms_norm_quant_nvfp4_swizzled_bf16` role). y is computed
 * exactly as in frt_ada_norm_quant_fp8, then block-quantised along each
 * row (blocks of 32 columns, dynamic scales).
 *
 *   M, D          rows; D a multiple of 256 in [512, 16384].
 *   residual, x, gate, weight, mod, eps, residual_out, gate_out   as in
 *                 frt_ada_norm_quant_fp8 (16-byte aligned, ld % 8 == 0).
 *   out_fp4       [M, ld_out] code bytes, ld_out >= D/2, a multiple of 4.
 *   out_scale     scale bytes [D/256][rows][8]; ld_sc = the run stride in
 *                 bytes, >= 8*M (8 * the buffer's row capacity).
 */
int frt_ada_norm_quant_mxfp4(void* stream, int64_t M, int64_t D,
                             const uint16_t* residual, int64_t ld_res,
                             const uint16_t* x, int64_t ld_x,
                             const uint16_t* gate, int64_t ld_gate,
                             const uint16_t* weight,
                             const uint16_t* mod, int64_t ld_mod, float eps,
                             uint16_t* residual_out, int64_t ld_rout,
                             uint8_t* out_fp4, int64_t ld_out,
                             uint8_t* out_scale, int64_t ld_sc,
                             uint16_t* gate_out, int64_t ld_gout);

/*
 * frt_packed_gemm_mxfp4_split — the packed GEMM on MXFP4 operands with the
 * bias + column-split epilogue. For m < M, n < N_total:
 *   acc[m, n] = sum_k dec(x[m, k]) * dec(W[n, k])   (block-scaled e2m1,
 *               the matrix cores' fp32 accumulation)
 *   out_s[m, n - off_s] = bf16_rne(acc[m, n] + bias_cat[n])   (or fp32)
 *
 *   M, K          rows; K a multiple of 256 in [512, 16384] (the
 *                 producer's D).
 *   x4, ld_x4     [M, ld_x4] code bytes (16-byte aligned, ld_x4 >= K/2, a
 *                 multiple of 16).
 *   xs, ld_xs     scale bytes [K/256][rows][8], ld_xs the run stride
 *                 (>= 8*M, a multiple of 4; 4-byte aligned), as
 *                 frt_ada_norm_quant_mxfp4 writes.
 *   W4, S4        [N_total, K/2] codes (16-byte aligned) and the scales
 *                 [K/256][N_total][8] (4-byte aligned), as
 *                 frt_pack_weights_mxfp4 writes.
 *   bias_cat, n_split, split_n, out, ld_out, out_dtype   as in
 *                 frt_packed_gemm_fp8_split (outputs must not overlap the
 *                 operands or the scales).
 */
int frt_packed_gemm_mxfp4_split(void* stream, int64_t M, int64_t K,
                                const uint8_t* x4, int64_t ld_x4,
                                const uint8_t* xs, int64_t ld_xs,
                                const uint8_t* W4, const uint8_t* S4,
                                int64_t N_total, const uint16_t* bias_cat,
                                int n_split, const int64_t* split_n,
                                void* const* out, const int64_t* ld_out,
                                int out_dtype);

/*
 * frt_packed_gemm_mxfp4_geglu_quant — the merged gate/up GEMM on MXFP4
 * operands with the GEGLU quantiser as its epilogue: the FFN tail of the
 * 4-bit band (fp8_chain.py `BANDS`: the norm-fed gate/up projection in the
 * block-scaled 4-bit format, the down projection kept in static FP8, so the
 * GEGLU output is quantised to e4m3fn for it). For m < M, j < H, with acc
 * as in frt_packed_gemm_mxfp4_split over W4 rows j (gate) and H + j (up):
 *   g = bf16_rne(acc[m, j] + bias_cat[j]),  u = bf16_rne(acc[m, H + j] + bias_cat[H + j])
 *   out_fp8[m, j] = e4m3_rne(clamp(fl32(gelu_tanh(g) * u / out_scale), +-448))
 * i.e. exactly frt_packed_gemm_mxfp4_split (bf16 out) followed by
 * frt_geglu_quant_fp8 on its output.
 *
 *   M, K, x4, ld_x4, xs, ld_xs   as in frt_packed_gemm_mxfp4_split.
 *   W4, S4        [2H, K/2] codes and [K/256][2H][8] scales: the H gate
 *                 rows, then the H up rows (frt_pack_weights_mxfp4 of the
 *                 siblings {gate, up}).
 *   H             width of each half (1 <= H, 2H <= 2^24).
 *   bias_cat      bf16 [2H] or NULL.
 *   out_scale     fp32 [1] (> 0): the down projection's static input scale.
 *   out_fp8       e4m3fn [M, ld_out], ld_out >= H; must not overlap an
 *                 input.
 */
int frt_packed_gemm_mxfp4_geglu_quant(void* stream, int64_t M, int64_t K,
                                      const uint8_t* x4, int64_t ld_x4,
                                      const uint8_t* xs, int64_t ld_xs,
                                      const uint8_t* W4, const uint8_t* S4,
                                      int64_t H, const uint16_t* bias_cat,
                                      const float* out_scale, uint8_t* out_fp8,
                                      int64_t ld_out);

/*
 * frt_packed_gemm_mxfp4_geglu_mxfp4 — the MXFP4 gate/up GEMM with the GEGLU
 * quantised to MXFP4 in its epilogue: the 4-bit band's `fp4_full` row
 * (fp8_chain.py `BANDS`: the GELU-mul emits packed 4-bit codes and the down
 * projection runs in 4-bit), fused. For m < M, j < H, with g and u as in
 * frt_packed_gemm_mxfp4_geglu_quant and y = gelu_tanh(g) * u (fp32), y is
 * quantised as frt_geglu_quant_mxfp4 quantises it, i.e. the result equals
 * frt_packed_gemm_mxfp4_split (bf16 out) followed by frt_geglu_quant_mxfp4.
 *
 *   M, K, x4, ld_x4, xs, ld_xs, W4, S4, bias_cat   as in
 *                 frt_packed_gemm_mxfp4_geglu_quant.
 *   H             width of each half, a multiple of 256 (2H <= 2^24).
 *   out_fp4, ld_out, out_scale, ld_sc   as in frt_geglu_quant_mxfp4; must
 *                 not overlap an input or each other.
 */
int frt_packed_gemm_mxfp4_geglu_mxfp4(void* stream, int64_t M, int64_t K,
                                      const uint8_t* x4, int64_t ld_x4,
                                      const uint8_t* xs, int64_t ld_xs,
                                      const uint8_t* W4, const uint8_t* S4,
                                      int64_t H, const uint16_t* bias_cat,
                                      uint8_t* out_fp4, int64_t ld_out,
                                      uint8_t* out_scale, int64_t ld_sc);

/*
 * frt_quantize_mxfp4 — dynamic MXFP4 quantiser of a bf16 tensor: the 4-bit
 * band's quantize-from-bf16 entry (fp8_chain.py `BANDS`, the `fp4` row's
 * GEMM package; `PackedLinearNvfp4` quantises a bf16 input it does not get
 * from a producer), for GEMM inputs that no norm producer writes, such as
 * the attention output before the O projection. Per row m < M, block
 * b < D/32 of 32 columns:
 *   s = 2^(floor(log2 max_k |x[m, 32b + k]|) - 2)   (E8M0 byte; 0 for an
 *       all-zero block, 0xFF when the block holds a NaN or an infinity)
 *   code[m, 32b + k] = e2m1_rne(x[m, 32b + k] / s)  (saturating at +-6)
 * i.e. the OCP MX conversion of the bf16 values; both the scale and the
 * codes are decided on those exact values.
 *
 *   M, D          rows; D a multiple of 256 (1 <= D/256, D <= 2^24).
 *   x, ld_x       bf16 [M, ld_x], 16-byte aligned, ld_x >= D, ld_x % 8 == 0.
 *   out_fp4, ld_out   [M, ld_out] code bytes (element 2j in the low nibble),
 *                 4-byte aligned, ld_out >= D/2, ld_out % 4 == 0.
 *   out_scale, ld_sc  scale bytes [D/256][rows][8] (run stride ld_sc >= 8M),
 *                 each run's blocks in the order 0, 2, 4, 6, 1, 3, 5, 7 (the
 *                 layout frt_packed_gemm_mxfp4_split reads).
 * Outputs must not overlap the input or each other.
 */
int frt_quantize_mxfp4(void* stream, int64_t M, int64_t D,
                       const uint16_t* x, int64_t ld_x,
                       uint8_t* out_fp4, int64_t ld_out,
                       uint8_t* out_scale, int64_t ld_sc);

/*
 * frt_geglu_quant_mxfp4 — the GEGLU of a bf16 gate|up buffer quantised to
 * MXFP4: the 4-bit band's GELU-mul that emits packed 4-bit codes for a 4-bit
 * down projection (fp8_chain.py `BANDS`, the `fp4_full` row). For m < M,
 * j < H: y = gelu_tanh(gu[m, j]) * gu[m, H + j] (fp32, as
 * frt_geglu_quant_fp8 forms it), then y is quantised as frt_quantize_mxfp4
 * quantises x (blocks of 32 along H).
 *
 *   M, H          rows; width of each half, a multiple of 256 (2H <= 2^24).
 *   gu, ld_gu     bf16 [M, ld_gu]: gate in [0, H), up in [H, 2H); 16-byte
 *                 aligned, ld_gu >= 2H, ld_gu % 8 == 0.
 *   out_fp4, ld_out, out_scale, ld_sc   as in frt_quantize_mxfp4 (D = H).
 */
int frt_geglu_quant_mxfp4(void* stream, int64_t M, int64_t H,
                          const uint16_t* gu, int64_t ld_gu,
                          uint8_t* out_fp4, int64_t ld_out,
                          uint8_t* out_scale, int64_t ld_sc);

/*
 * frt_interleave_pairs_bf16 — the pack-time permutation of q or k
 * projection rows that turns the host's rotate-half rotary pairs
 * (i, i + hd/2) into adjacent pairs (2i, 2i + 1).
 *
 * Source: fp8_chain.py, module docstring (the two RoPE layouts and why a
 * shared permutation of the head dimension leaves attention unchanged),
 * `_quantize` (`_interleave_rows` on the q and k weights before packing;
 * V keeps host order) and the `kperm` gather (position 2i takes dimension
 * i, 2i + 1 takes i + hd/2). For h < nheads, j < hd, k < K:
 *   dst[h*hd + j, k] = src[h*hd + perm(j), k],
 *   perm(2i) = i, perm(2i + 1) = i + hd/2.
 *
 *   nheads, hd    heads and (even) head dim of the projection.
 *   K             row length (input width), >= 1.
 *   src, dst      bf16 [nheads*hd, K] row-packed; must not overlap.
 * Rows are copied bit for bit; apply it to the q and k siblings before
 * frt_pack_weights_fp8 when the GEMM feeds a RoPE consumer.
 */
int frt_interleave_pairs_bf16(void* stream, int nheads, int hd, int64_t K,
                              const uint16_t* src, uint16_t* dst);

/*
 * frt_qkv_split_rope_kvcache — split the merged QKV output, rotate q and k
 * by adjacent-pair RoPE, write q and the suffix rows of the K/V caches.
 *
 * Source: fp8_chain.py `_make_run` (`qkv_split_rope_kvcache_bf16(qkv3,
 * rope, nh, kv, hd, P, q_out=, k_cache=, v_cache=, max_seq_len=T)` with the
 * suffix K/V written behind P prefix rows, T = P + S), `_build_rope` (the
 * table layout) and the module docstring (adjacent pairs). For token m < S,
 * head h, pair i < hd/2, with (c, s) = (rope[m, 2i], rope[m, 2i + 1]):
 *   (a, b) = the pair's two values of q (or k) head h
 *   a' = bf16_rne(a c - b s),  b' = bf16_rne(b c + a s)
 *   q_out[m, h, :]      = rotated q head h
 *   k_cache[P + m, h, :] = rotated k head h   (h < kv)
 *   v_cache[P + m, h, :] = v head h, copied   (h < kv)
 * Cache rows outside [P, P + S) are not touched. Both products are exact
 * in fp32, so the rotated values are the single rounding of the exact
 * result (bit-exact to the definition).
 *
 *   S             tokens (rows of qkv; 0 => no-op).
 *   nh, kv, hd    query heads, KV heads (>= 1), even head dim.
 *   qkv           bf16 [S, ld_qkv], columns q (nh*hd) | k (kv*hd) |
 *                 v (kv*hd); q and k pair-interleaved (see
 *                 frt_interleave_pairs_bf16). 4-byte aligned, ld even.
 *   rope          bf16 [S, hd]: cos at even, sin at odd columns. 4-byte
 *                 aligned.
 *   P, T          first cache row written and the caches' rows (P + S <= T).
 *   q_out         bf16 [S, nh, hd] contiguous.
 *   k_cache, v_cache   bf16 [T, kv, hd] contiguous.
 * Outputs must not overlap each other, qkv or rope. hd % 8 == 0 with every
 * pointer 16-byte aligned and ld_qkv % 8 == 0 takes the vector path.
 */
int frt_qkv_split_rope_kvcache(void* stream, int64_t S, int nh, int kv,
                               int hd, const uint16_t* qkv, int64_t ld_qkv,
                               const uint16_t* rope, int64_t P, int64_t T,
                               uint16_t* q_out, uint16_t* k_cache,
                               uint16_t* v_cache);

/*
 * frt_packed_gemm_fp8_qkv_rope — the merged QKV FP8 GEMM with the split +
 * RoPE + KV-cache write as its epilogue (the bf16 QKV buffer never reaches
 * memory).
 *
 * Source: as frt_packed_gemm_fp8_split for the GEMM and
 * frt_qkv_split_rope_kvcache for the consumer. For m < M and column n of
 * the [M, (nh + 2kv) hd] product:
 *   v = bf16_rne(fl32(alpha * acc[m, n]) + bias_cat[n])
 * then exactly frt_qkv_split_rope_kvcache on those values (token m = row
 * m), i.e. the same results as frt_packed_gemm_fp8_split (bf16 out)
 * followed by frt_qkv_split_rope_kvcache.
 *
 *   M, K, x8, ld_x, act_scale, w_scale, bias_cat   as in
 *                 frt_packed_gemm_fp8_split (bias_cat [(nh + 2kv) hd]).
 *   W8            e4m3fn [(nh + 2kv) hd, K]: q rows, k rows (both
 *                 pair-interleaved before packing), v rows.
 *   nh, kv, hd, rope, P, T, q_out, k_cache, v_cache   as in
 *                 frt_qkv_split_rope_kvcache (S = M).
 */
int frt_packed_gemm_fp8_qkv_rope(void* stream, int64_t M, int64_t K,
                                 const uint8_t* x8, int64_t ld_x,
                                 const uint8_t* W8, int nh, int kv, int hd,
                                 const float* act_scale,
                                 const float* w_scale,
                                 const uint16_t* bias_cat,
                                 const uint16_t* rope, int64_t P, int64_t T,
                                 uint16_t* q_out, uint16_t* k_cache,
                                 uint16_t* v_cache);

/*
 * frt_packed_gemm_mxfp4_qkv_rope — the merged QKV GEMM on MXFP4 operands
 * with the split + RoPE + KV-cache write as its epilogue: the 4-bit band's
 * QKV projection feeding the attention head. For m < M and column n of the
 * [M, (nh + 2kv) hd] product:
 *   v = bf16_rne(acc[m, n] + bias_cat[n])   (acc as in
 *       frt_packed_gemm_mxfp4_split)
 * then exactly frt_qkv_split_rope_kvcache on those values, i.e. the same
 * results as frt_packed_gemm_mxfp4_split (bf16 out) followed by
 * frt_qkv_split_rope_kvcache.
 *
 *   M, K, x4, ld_x4, xs, ld_xs   as in frt_packed_gemm_mxfp4_split.
 *   W4, S4        [(nh + 2kv) hd, K/2] codes and [K/256][(nh + 2kv) hd][8]
 *                 scales: q rows, k rows (both pair-interleaved before
 *                 packing, frt_interleave_pairs_bf16), v rows.
 *   bias_cat      bf16 [(nh + 2kv) hd] or NULL.
 *   nh, kv, hd, rope, P, T, q_out, k_cache, v_cache   as in
 *                 frt_qkv_split_rope_kvcache (S = M).
 */
int frt_packed_gemm_mxfp4_qkv_rope(void* stream, int64_t M, int64_t K,
                                   const uint8_t* x4, int64_t ld_x4,
                                   const uint8_t* xs, int64_t ld_xs,
                                   const uint8_t* W4, const uint8_t* S4,
                                   int nh, int kv, int hd,
                                   const uint16_t* bias_cat,
                                   const uint16_t* rope, int64_t P, int64_t T,
                                   uint16_t* q_out, uint16_t* k_cache,
                                   uint16_t* v_cache);

#ifdef __cplusplus
}
#endif

#endif /* FRT_H_ */
