/*
 * ffn.h — C ABI of libffn.so: the forward hot path of a Llama-style dense
 * SwiGLU FFN block and its FP8 single-token decode form, on AMD MI355X (gfx950).
 *
 * Conventions for every entry point
 *   - Every pointer is DEVICE memory (hipMalloc / torch CUDA tensors) unless
 *     stated otherwise.  The caller allocates and owns every buffer; the library
 *     allocates nothing and keeps no state between calls.
 *   - Every call is asynchronous on `stream` (0 = the null stream).  Results are
 *     valid once the stream has been synchronised; no call synchronises.
 *   - Matrices are row-major and contiguous.  Weights are [out, in], so both
 *     operands of every matmul are contiguous along the reduction dimension.
 *   - bf16 = IEEE binary32 truncated to 16 bits (round to nearest even);
 *     e4m3 = OCP E4M3FN (max 448, NaN 0x7F/0xFF, no infinities).
 *   - Abs-max outputs are OVERWRITTEN with max|x| of the tensor just written
 *     (the library clears them itself on `stream` first), except in the
 *     calls whose names end in _acc, which max-accumulate into a word the
 *     caller has zeroed (the convention of [llmq model] LLamaModel::forward:
 *     the abs-max table, whose slots include the backward's gradients, is
 *     zeroed once and every producer accumulates into its slot), and
 *     ffn_quant_absmax_clear, ffn_quant_transpose_clear and
 *     ffn_rmsnorm_bwd_acc, which zero a slot for its next producer.
 *     Abs-max is the maximum of |x| over the bit patterns, so a NaN element
 *     makes it NaN (and every code of the tensor a NaN code).
 *   - A dequantisation scale is absmax/448 (1.0 when absmax == 0); codes are
 *     e4m3(x * (448/absmax)), with the product taken in fp32, rounded to
 *     nearest even and saturated at +-448.
 *   - Errors are return values.  Arguments are validated before any HIP call:
 *     a NULL required pointer, a negative size or an unknown enum gives
 *     FFN_ERR_INVALID; a size the kernels do not support, or a pointer not
 *     aligned to 16 bytes, gives FFN_ERR_UNSUPPORTED; a failed launch gives
 *     FFN_ERR_HIP.  Nothing is launched when validation fails.  A zero row
 *     count (N or M == 0) is valid and writes no rows; the per-tensor outputs
 *     keep their meaning (an abs-max of no elements is 0, accumulated ones
 *     stay as found, scales are still written from their abs-max, dweight
 *     stays as found).  ffn_last_error()
 *     returns a thread-local description of the last non-OK status.
 *   - Calls that share an output buffer on different streams race; calls on one
 *     stream are ordered.
 *   - Size limits (FFN_ERR_UNSUPPORTED beyond them): each input operand of a
 *     GEMM (ffn_gateup, ffn_gateup_swiglu_quant, ffn_down, ffn_matmul_tn,
 *     ffn_matmul_tn_swiglu_bwd) is under 4 GiB and its row count under
 *     2^31 - 256 (the kernels keep byte offsets inside one operand in 32 bits;
 *     outputs may be larger); each decode weight matrix is under 2 GiB; row
 *     counts of the row-wise kernels are at most 2^31; ffn_quant_absmax,
 *     ffn_swiglu and ffn_swiglu_bwd take up to 2^36 elements.
 *
 * Citations name the page and the function on it that defines the operation:
 *   [llmq model]  IST-DASLab llmq, src/models/llama_model.cpp
 *   [llmq state]  IST-DASLab llmq, src/models/llama_run_state.cpp
 *   [metrale]     metrale_model_layers/layers/dense_ffn_decode.rs
 */
#ifndef FFN_H
#define FFN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
    FFN_OK = 0,
    FFN_ERR_INVALID = 1,      /* NULL required pointer, negative size, bad enum   */
    FFN_ERR_UNSUPPORTED = 2,  /* size / alignment outside what the kernels handle */
    FFN_ERR_HIP = 3           /* a HIP launch or runtime call failed               */
} ffn_status_t;

typedef enum {
    FFN_BF16 = 0,             /* bf16 operands, no scales                          */
    FFN_E4M3 = 1,             /* e4m3 operands with per-tensor fp32 scales         */
    FFN_E5M2 = 2              /* e5m2 gradient codes (scale absmax / 57344) beside
                                 e4m3 weights and activations: the backward's other
                                 FP8 grad dtype                                     */
} ffn_dtype_t;

/* Fused residual add + RMSNorm, saving rstd, with the output's abs-max.
 * [llmq model] LLamaModel::_forward_block, fused_residual_rmsnorm_forward
 * (residual stream + attention output -> LN2, LN2_Rstd, LN2 abs-max);
 * LLamaModel::forward, rmsnorm_forward for the form without a residual.
 * [llmq state] allocate_basic_fwd_tensors: rstd is fp32 [B,T]; the norm output
 * may overwrite its input.
 *
 *   r      = bf16(inp + addend)                 -> residual_out   (bf16 [N,C])
 *   rstd_i = 1 / sqrt(sum_j r_ij^2 / C + eps)   -> rstd           (fp32 [N])
 *   y      = bf16(r * rstd * weight)            -> y              (bf16 [N,C])
 *   max|y|                                      -> absmax         (fp32 [1])
 *
 * addend == NULL: plain RMSNorm, r = inp, residual_out must be NULL.
 * absmax may be NULL (not computed).  y may alias inp or addend (each row is
 * read completely before it is written); residual_out may alias inp.
 * Supported: C % 8 == 0, 8 <= C <= 16384.  N >= 0. */
ffn_status_t ffn_rmsnorm_fwd(void* y, float* rstd, void* residual_out, float* absmax,
                             const void* inp, const void* addend, const void* weight,
                             float eps, int64_t N, int64_t C, hipStream_t stream);

/* Per-tensor abs-max FP8 e4m3 quantisation of a bf16 tensor of n elements.
 * [llmq model] forward_qmm, quantize_with_abs_max(inp.Quant, inp.Quant.scale(),
 * inp.Value, inp.Quant.abs_max(), B*T*C); LLamaModel::_forward_block, abs_max.
 * [llmq state] allocate_fwd_quant_tensors: e4m3 copies, fp32 abs-max and scale.
 *
 *   compute_absmax != 0: *absmax = max|x| is computed first (overwritten);
 *   compute_absmax == 0: *absmax is read as given (e.g. from ffn_rmsnorm_fwd
 *                        or the fused ffn_gateup epilogue).
 *   *scale = absmax/448 (1 if absmax == 0);  q = e4m3(x * 448/absmax).
 * q: e4m3 [n]; x: bf16 [n]; scale, absmax: fp32 [1].  Any n >= 0. */
ffn_status_t ffn_quant_absmax(uint8_t* q, float* scale, float* absmax, const void* x,
                              int64_t n, int compute_absmax, hipStream_t stream);

/* ffn_rmsnorm_fwd that max-accumulates max|y| into *absmax (required) as
 * found, without clearing it first: the caller zeroes the word once (at
 * allocation, or through ffn_quant_absmax_clear) rather than before every
 * producer.  [llmq model] LLamaModel::forward zeroes the abs-max table once
 * per forward (fill_zero) and every quantised tensor's producer accumulates
 * into its slot.  Other arguments and results as ffn_rmsnorm_fwd. */
ffn_status_t ffn_rmsnorm_fwd_acc(void* y, float* rstd, void* residual_out, float* absmax,
                                 const void* inp, const void* addend, const void* weight,
                                 float eps, int64_t N, int64_t C, hipStream_t stream);

/* ffn_quant_absmax with the abs-max given (compute_absmax == 0) that also sets
 * *clear = 0: the abs-max slot of a tensor whose consumer has run and whose
 * producer (an _acc call) comes later on the stream.  [llmq model]
 * LLamaModel::forward (the table's zeroing), forward_qmm
 * (quantize_with_abs_max).  In the block's forward the quantiser of y clears
 * h's slot and the quantiser of h clears y's slot for the next forward, so
 * the table, zeroed once at allocation, needs no clearing launch.  clear must
 * be a word other than scale and absmax.  Other arguments as
 * ffn_quant_absmax. */
ffn_status_t ffn_quant_absmax_clear(uint8_t* q, float* scale, const float* absmax, const void* x,
                                    int64_t n, float* clear, hipStream_t stream);

/* Per-row abs-max e4m3 quantisation of a bf16 weight [rows, cols]: the
 * QuantizedWeight { weight, row_scale } layout the FP8 decode consumes.
 * [metrale] DenseFfnLayer::forward, FP8 arm (gate_proj/up_proj/down_proj
 * weight + row_scale).  An offline weight-preparation step, not part of the
 * per-token path.  q: e4m3 [rows, cols]; row_scale: fp32 [rows].
 * Supported: cols % 8 == 0. */
ffn_status_t ffn_quant_rows(uint8_t* q, float* row_scale, const void* w,
                            int64_t rows, int64_t cols, hipStream_t stream);

/* Fused gate+up projection, optionally with the SwiGLU epilogue.
 * [llmq model] LLamaModel::_forward_block, forward_qmm(MlpUp, LN2, MLP_Up_w,
 * B, T, C, 2*D) and swiglu_forward; forward_qmm: matmul TN, scaled by
 * weight.scale() and inp.Quant.scale() when the operands are FP8.
 *
 *   GU[n,o] = sum_k x[n,k] * w[o,k]  (* x_scale * w_scale for E4M3), o < 2H,
 *   rows [0,H) of w are the gate, rows [H,2H) the up projection.
 *   fuse_swiglu == 0: out = bf16(GU)                      bf16 [N, 2H]
 *   fuse_swiglu != 0: out = bf16(silu(g) * u), g = bf16(GU[:, :H]),
 *                     u = bf16(GU[:, H:])                 bf16 [N, H]
 *   out_absmax (nullable) = max|out|.
 * x: bf16 or e4m3 [N,C]; w: same dtype [2H,C]; x_scale, w_scale: fp32 [1],
 * required for E4M3, ignored for BF16.  fp32 accumulation.
 * Supported: C % 128 == 0, H % 128 == 0, N >= 0. */
ffn_status_t ffn_gateup(void* out, float* out_absmax, const void* x, const float* x_scale,
                        const void* w, const float* w_scale, ffn_dtype_t dtype, int fuse_swiglu,
                        int64_t N, int64_t C, int64_t H, hipStream_t stream);

/* ffn_gateup with the SwiGLU epilogue (fuse_swiglu = 1) that max-accumulates
 * max|h| into *h_absmax (required) as found, as ffn_rmsnorm_fwd_acc does.
 * h: bf16 [N, H]; other arguments as ffn_gateup; h_absmax must not alias the
 * scales. */
ffn_status_t ffn_gateup_acc(void* h, float* h_absmax, const void* x, const float* x_scale,
                            const void* w, const float* w_scale, ffn_dtype_t dtype,
                            int64_t N, int64_t C, int64_t H, hipStream_t stream);

/* Fused gate+up projection with the SwiGLU epilogue storing e4m3 codes of h
 * quantised with an abs-max known beforehand (one pass instead of bf16 h, then
 * ffn_quant_absmax).  [llmq model] LLamaModel::_recompute_block:
 * swiglu_forward_quant(SwiGLu.Quant, its scale, MlpUp, its abs-max), which
 * re-creates the quantised SwiGLU output under the abs-max the forward pass
 * recorded; forward_qmm with reuse_inp_quant then feeds it to the down GEMM.
 *
 *   h = bf16(silu(g) * u) exactly as ffn_gateup with fuse_swiglu;
 *   *q_scale = A/448 (1 if A == 0),  q = e4m3(h * 448/A),  A = *h_absmax_known;
 *   h_absmax (nullable) = max|h| of this call's h (e.g. the next call's A).
 * q is bit-identical to ffn_gateup(fuse_swiglu) followed by
 * ffn_quant_absmax(compute_absmax = 0) with absmax = A; values beyond A
 * saturate to +-448.
 * q: e4m3 [N,H]; q_scale, h_absmax, h_absmax_known: fp32 [1]; x, w, scales as
 * ffn_gateup.  h_absmax_known is required and must differ from h_absmax and
 * q_scale (both are written while it is read).  Supported: C % 128 == 0,
 * H % 128 == 0, N >= 0. */
ffn_status_t ffn_gateup_swiglu_quant(uint8_t* q, float* q_scale, float* h_absmax,
                                     const float* h_absmax_known, const void* x, const float* x_scale,
                                     const void* w, const float* w_scale, ffn_dtype_t dtype,
                                     int64_t N, int64_t C, int64_t H, hipStream_t stream);

/* SwiGLU on an unfused gate+up output, with the output's abs-max.
 * [llmq model] LLamaModel::_forward_block, swiglu_forward(SwiGLu, MlpUp,
 * SwiGLu abs-max, B, T, D).  h = bf16(silu(g) * u), g = gu[:, :H], u = gu[:, H:].
 * h: bf16 [N,H]; gateup: bf16 [N,2H]; absmax nullable.  Supported: H % 8 == 0. */
ffn_status_t ffn_swiglu(void* h, float* absmax, const void* gateup,
                        int64_t N, int64_t H, hipStream_t stream);

/* Down projection.  [llmq model] LLamaModel::_forward_block,
 * forward_qmm(MlpDown, SwiGLu, MLP_Down_w, B, T, D, C).
 *   out[n,c] = bf16(sum_j h[n,j] * w[c,j]  (* h_scale * w_scale for E4M3))
 * out: bf16 [N,C]; h: bf16 or e4m3 [N,H]; w: same dtype [C,H]; scales fp32 [1]
 * (E4M3 only).  Supported: C % 128 == 0, H % 128 == 0. */
ffn_status_t ffn_down(void* out, const void* h, const float* h_scale,
                      const void* w, const float* w_scale, ffn_dtype_t dtype,
                      int64_t N, int64_t H, int64_t C, hipStream_t stream);

/* ---------------------------------------------------------- tiled operands
 * The prefill products on operands stored in this library's tiled layout
 * instead of row-major: the same products as ffn_gateup_acc,
 * ffn_gateup_swiglu_quant and ffn_down (bit for bit: the same sums in the
 * same order), with every global load of the GEMM reading one contiguous
 * KiB.  The pages fix only the row-major tensors; the layout is a storage
 * choice of this library, made once for the weights (ffn_tile_pack) and by
 * the quantisers for the activations.
 *
 * Layout of a [R, K] operand (K bytes per row, K % 64 == 0; e4m3 codes or
 * bf16 values alike): rows in groups of 64, group g at byte g*64*K; inside
 * a group, K-step s (bytes 64s .. 64s+63 of each row) at s*4096, and its
 * 16-row sub-group i at + i*1024; there, lane l = 0..63 holds 16 bytes at
 * + 16*l: bytes 16*((l % 4) XOR (l / 16)) .. +15 of K-step s of row
 * 64g + 16i + l/4.  A tiled buffer holds whole groups: ffn_tile_bytes(R, K)
 * = ceil(R/64)*64*K bytes; the rows past R in the last group are don't-care
 * for the GEMMs (a token row only feeds its own output row, which is
 * neither stored nor counted in an abs-max). */

/* Bytes of the tiled form of [rows, row_bytes] (-1 if row_bytes % 64 != 0
 * or a size is negative). */
int64_t ffn_tile_bytes(int64_t rows, int64_t row_bytes);

/* Tiled copy of a row-major [rows, row_bytes] operand (the weights, once per
 * update); rows past `rows` in the last group are written as zeros.  out:
 * ffn_tile_bytes(rows, row_bytes) bytes, must not overlap in.  Supported:
 * row_bytes % 64 == 0, 64 <= row_bytes <= 2^21, the tiled size < 2^36. */
ffn_status_t ffn_tile_pack(void* out, const void* in, int64_t rows, int64_t row_bytes,
                           hipStream_t stream);

/* ffn_quant_absmax_clear for a [rows, cols] bf16 x whose codes are stored in
 * the tiled layout (the same codes, moved): *scale = A/448 (1 if A == 0),
 * q = e4m3(x * 448/A), A = *absmax; clear (nullable) is zeroed.  q:
 * ffn_tile_bytes(rows, cols) bytes (rows past `rows` are left as found),
 * must not overlap x.  Supported: cols % 128 == 0, cols <= 2^20,
 * ffn_tile_bytes(rows, cols) <= 2^36. */
ffn_status_t ffn_quant_absmax_clear_tiled(uint8_t* q, float* scale, const float* absmax,
                                          const void* x, int64_t rows, int64_t cols, float* clear,
                                          hipStream_t stream);

/* ffn_gateup_acc (E4M3) with x [N, C] and w [2H, C] tiled; h bf16 [N, H]
 * row-major.  [llmq model] LLamaModel::_forward_block, forward_qmm and
 * swiglu_forward.  Supported as ffn_gateup_acc, and ffn_tile_bytes(N, C) <
 * 2^32. */
ffn_status_t ffn_gateup_acc_tiled(void* h, float* h_absmax, const uint8_t* x, const float* x_scale,
                                  const uint8_t* w, const float* w_scale, int64_t N, int64_t C,
                                  int64_t H, hipStream_t stream);

/* ffn_gateup_swiglu_quant (E4M3) with x and w tiled and the codes q of h
 * stored tiled [N, H] (ffn_tile_bytes(N, H) bytes; rows past N are not
 * written).  [llmq model] LLamaModel::_recompute_block,
 * swiglu_forward_quant.  Supported as ffn_gateup_swiglu_quant. */
ffn_status_t ffn_gateup_swiglu_quant_tiled(uint8_t* q, float* q_scale, float* h_absmax,
                                           const float* h_absmax_known, const uint8_t* x,
                                           const float* x_scale, const uint8_t* w,
                                           const float* w_scale, int64_t N, int64_t C, int64_t H,
                                           hipStream_t stream);

/* ffn_down (E4M3) with h [N, H] and w [C, H] tiled; out bf16 [N, C]
 * row-major.  [llmq model] LLamaModel::_forward_block, forward_qmm(MlpDown,
 * ...).  Supported as ffn_down, and ffn_tile_bytes(N, H) < 2^32. */
ffn_status_t ffn_down_tiled(void* out, const uint8_t* h, const float* h_scale, const uint8_t* w,
                            const float* w_scale, int64_t N, int64_t H, int64_t C,
                            hipStream_t stream);

/* The bf16 block on tiled operands.  ffn_rmsnorm_fwd with y [N, C] bf16
 * stored tiled (rows of 2C bytes: ffn_tile_bytes(N, 2C) bytes; rows past N
 * are left as found; y must not overlap inp, addend or residual_out, and
 * C % 32 == 0); ffn_gateup (BF16, fuse_swiglu = 1) with x [N, C] and w
 * [2H, C] tiled and h [N, H] stored tiled (out_absmax nullable, as there);
 * ffn_down (BF16) with h and w [C, H] tiled and out row-major.  [llmq model]
 * LLamaModel::_forward_block (fused_residual_rmsnorm_forward, forward_qmm,
 * swiglu_forward).  Results equal the row-major calls' bit for bit.
 * Supported as the row-major calls, and each tiled operand < 4 GiB. */
ffn_status_t ffn_rmsnorm_fwd_tiled(void* y, float* rstd, void* residual_out, float* absmax,
                                   const void* inp, const void* addend, const void* weight,
                                   float eps, int64_t N, int64_t C, hipStream_t stream);
ffn_status_t ffn_gateup_tiled_bf16(void* h, float* h_absmax, const void* x, const void* w,
                                   int64_t N, int64_t C, int64_t H, hipStream_t stream);
ffn_status_t ffn_down_tiled_bf16(void* out, const void* h, const void* w, int64_t N, int64_t H,
                                 int64_t C, hipStream_t stream);

/* FP8-weight, bf16-activation decode FFN for M tokens (split-SiLU arm).
 * [metrale] DenseFfnLayer::forward, FP8 arm: w8a16_gemv_dual (gate and up in
 * one pass, per-row scales), silu_mul in place, w8a16_gemv for the down
 * projection.  The SiLU * up product is fused into the dual GEMV's epilogue.
 *
 *   g = bf16(s_gate[n] * sum_k w_gate[n,k] x[m,k]),  u likewise,
 *   h = bf16(silu(g) * u)                                    -> h   bf16 [M,H]
 *   out[m,c] = bf16(s_down[c] * sum_n w_down[c,n] h[m,n])    -> out bf16 [M,C]
 * x: bf16 [M,C]; w_gate, w_up: e4m3 [H,C]; w_down: e4m3 [C,H];
 * s_gate, s_up: fp32 [H]; s_down: fp32 [C].  h is caller-provided and also
 * returned.  Supported: 0 <= M <= 32, C % 128 == 0, H % 128 == 0. */
ffn_status_t ffn_decode_gemv(void* out, void* h, const void* x,
                             const uint8_t* w_gate, const float* s_gate,
                             const uint8_t* w_up, const float* s_up,
                             const uint8_t* w_down, const float* s_down,
                             int64_t M, int64_t C, int64_t H, hipStream_t stream);

/* The arms of the FP8 decode FFN.  [metrale] DenseFfnLayer::forward, FP8 arm,
 * and the note beside it: the split-SiLU arm (the default, ffn_decode_gemv)
 * forms silu(g) * u once before the down GEMV; the fused SiLU-input arm
 * (w8a16_gemv_silu_input) forms it inside the down GEMV, recomputing it for
 * every output; the per-projection arm runs gate and up as two GEMVs, then
 * silu_mul, then the down GEMV. */
typedef enum {
    FFN_DECODE_SPLIT_SILU = 0,
    FFN_DECODE_SILU_INPUT = 1,
    FFN_DECODE_PER_PROJECTION = 2
} ffn_decode_arm_t;

/* ffn_decode_gemv through a chosen arm.  All arms compute the same rounded
 * quantities (g, u and h = bf16(silu(g) * u) in bf16, the down GEMV on h), so
 * out is bit-identical across arms; only the kernels differ.
 * gu: bf16 [M, 2H] workspace (g in columns [0,H), u in [H,2H)), required by the
 * SiLU-input and per-projection arms, ignored by the split arm; h: bf16 [M,H],
 * written by the split and per-projection arms (the SiLU-input arm never forms
 * it).  Other arguments as ffn_decode_gemv.  Supported: M <= 32 for the split
 * arm, M <= 4 for the others; gu must not alias x, out or h. */
ffn_status_t ffn_decode_gemv_arm(void* out, void* h, void* gu, const void* x,
                                 const uint8_t* w_gate, const float* s_gate,
                                 const uint8_t* w_up, const float* s_up,
                                 const uint8_t* w_down, const float* s_down,
                                 ffn_decode_arm_t arm, int64_t M, int64_t C, int64_t H,
                                 hipStream_t stream);

/* Decode FFN with bf16 weights (no quantisation).  [metrale]
 * DenseFfnLayer::forward, bf16 arm: dense_gemv for gate and up, silu_mul,
 * dense_gemv for the down projection.
 *   g = bf16(sum_k w_gate[n,k] x[m,k]),  u likewise,  h = bf16(silu(g) * u),
 *   out[m,c] = bf16(sum_n w_down[c,n] h[m,n]).
 * x: bf16 [M,C]; w_gate, w_up: bf16 [H,C]; w_down: bf16 [C,H]; h: bf16 [M,H]
 * workspace, returned.  Supported: 0 <= M <= 4, C % 128 == 0, H % 128 == 0. */
ffn_status_t ffn_decode_gemv_bf16(void* out, void* h, const void* x,
                                  const void* w_gate, const void* w_up, const void* w_down,
                                  int64_t M, int64_t C, int64_t H, hipStream_t stream);

/* Packed decode weights: the same e4m3 codes re-laid so that the few-token
 * decode (faster than on row-major weights from three tokens on, up to 32)
 * reads one KiB (16 rows x 64 codes) per load instruction, in the order the
 * MFMA consumes it, and its waves, each walking its own 16-row blocks along
 * K, read neighbouring KiBs at any one moment (piece-major).
 * packed: e4m3, rows * cols bytes; 16-byte piece p holds row 16 rb + l % 16,
 * codes 64 kc + 16 (l / 16) .. + 15 of w, where l = p % 64 and
 * p / 64 = kc * (rows / 16) + rb.  A one-time re-layout of the QuantizedWeight
 * rows of [metrale] DenseFfnLayer::forward (FP8 arm); the row scales are
 * unchanged.  Supported: rows % 16 == 0, cols % 128 == 0; packed must not
 * alias w. */
ffn_status_t ffn_decode_pack_weight(uint8_t* packed, const uint8_t* w, int64_t rows,
                                    int64_t cols, hipStream_t stream);

/* Workspace bytes of ffn_decode_gemv_packed for M tokens; -1 for sizes it
 * does not support.  Up to 16 tokens: 32 (C + H) bytes (x and h in the MFMA's
 * operand order) plus 64 S C bytes of fp32 partial sums of the down
 * projection, which is split along its reduction dimension H into
 * S = max(1, min(H/64, max(256 / (C/128), ceil(H/64 / 64)))) slices (a
 * function of the shape alone, so results do not depend on the device);
 * 17 to 32 tokens: the larger of that and 64 (C + H) bytes.  Never smaller
 * for more tokens, so a workspace sized for the largest batch serves every
 * smaller one. */
int64_t ffn_decode_packed_workspace_bytes(int64_t M, int64_t C, int64_t H);

/* The split-SiLU decode of ffn_decode_gemv (same formulas, same results up to
 * fp32 summation order) on packed weights: w_gate, w_up [H, C] and w_down
 * [C, H] in the layout of ffn_decode_pack_weight; scales, x, h and out as in
 * ffn_decode_gemv.  workspace: ffn_decode_packed_workspace_bytes(M, C, H)
 * bytes, 16-byte aligned, caller-owned, any contents; it receives h (and,
 * above 16 tokens or C > 4096, x) in the order of the MFMA's activation
 * operand and, up to 16 tokens, the down projection's partial sums over its
 * S slices, added in slice order (all written and read within the call).
 * Supported: 0 <= M <= 32, C % 128 == 0, H % 128 == 0; the workspace must not
 * alias out, h or x.  Calls that share a workspace must not overlap. */
ffn_status_t ffn_decode_gemv_packed(void* out, void* h, void* workspace, const void* x,
                                    const uint8_t* w_gate, const float* s_gate,
                                    const uint8_t* w_up, const float* s_up,
                                    const uint8_t* w_down, const float* s_down,
                                    int64_t M, int64_t C, int64_t H, hipStream_t stream);

/* ffn_decode_gemv_packed without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace),
 * kernels and results as ffn_decode_gemv_packed; the workspace is a built-in
 * device array of ffn_decode_noalloc_scratch_bytes() bytes (8 MiB) that every
 * call on a device shares and that keeps the last call's contents (nothing in
 * it needs to start at zero).  Calls that overlap on one device (on different
 * streams, or from different threads) race on it; calls on one stream are
 * ordered.  Sizes whose ffn_decode_packed_workspace_bytes exceed it give
 * FFN_ERR_UNSUPPORTED.  The call allocates nothing: on its first use on a
 * device it looks up the array's device address (hipGetSymbolAddress). */
int64_t ffn_decode_noalloc_scratch_bytes(void);
ffn_status_t ffn_decode_gemv_packed_noalloc(void* out, void* h, const void* x,
                                            const uint8_t* w_gate, const float* s_gate,
                                            const uint8_t* w_up, const float* s_up,
                                            const uint8_t* w_down, const float* s_down,
                                            int64_t M, int64_t C, int64_t H, hipStream_t stream);

/* ------------------------------------------------------------------ backward
 * The FFN half of [llmq model] LLamaModel::_backward_block, as the calls it
 * is made of: backward_qmm through the down projection, swiglu_backward,
 * backward_qmm through the [2H, C] up weight, rmsnorm_backward.  backward_qmm
 * with e4m3 weights quantises the output gradient with its abs-max,
 * transposes the weight, the input codes and the gradient codes, and runs two
 * scaled TN matmuls; ffn_matmul_tn is that matmul (with bf16 operands as well)
 * and ffn_transpose / ffn_quant_transpose the transposes. */

/* Flags of the TN products.  FFN_TN_ACCUMULATE: add to out (see below).
 * FFN_TN_TILE_GRID: launch one workgroup per 256 x 256 output tile instead of
 * a persistent grid sized to the CUs, so that the hardware hands CUs to work
 * on other streams as tiles finish: for two independent products issued on
 * two streams (the data and weight gradients of one projection), whose partial
 * last rounds of tiles then fill each other.  Results do not depend on it.
 * FFN_TN_TILED (FP8 only): a and b are in the tiled layout (see the tiled
 * operands below: whole 64-row groups), the output row-major; the results
 * equal the row-major operands' bit for bit. */
#define FFN_TN_ACCUMULATE 1
#define FFN_TN_TILE_GRID 2
#define FFN_TN_TILED 4

/* TN matmul: out[m,n] = bf16(acc + sum_k a[m,k] * b[n,k] (* a_scale * b_scale
 * for FP8)), acc = out[m,n] when flags has FFN_TN_ACCUMULATE (the
 * accumulate_gradient flag of backward_qmm: one rounding of the fp32 sum),
 * else 0; FFN_TN_TILE_GRID and FFN_TN_TILED as above; other flag bits are
 * invalid.  [llmq model]
 * backward_qmm, matmul(..., EMMTranspose::TN, accumulate_gradient); the
 * gradient operand is allocated in the grad dtype (e4m3 or e5m2), the weight
 * and activation operands in e4m3.
 * out: bf16 [M,N]; a: [M,K], b: [N,K]; dtype FFN_BF16: both bf16, FFN_E4M3:
 * both e4m3, FFN_E5M2: a e5m2 (the gradient), b e4m3; scales fp32 [1] (FP8
 * only).  Supported: K % 128 == 0, N % 128 == 0, any M >= 0; out must not
 * alias a or b. */
ffn_status_t ffn_matmul_tn(void* out, const void* a, const float* a_scale,
                           const void* b, const float* b_scale, ffn_dtype_t dtype,
                           int flags, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream);

/* TN matmul fused with the SwiGLU backward: dh = bf16(sum_k a[m,k] * b[n,k]
 * (* a_scale * b_scale for FP8)) as ffn_matmul_tn would store it, then,
 * without storing dh, dgu = the gradient of h = silu(g) * u as
 * ffn_swiglu_bwd computes it from dh and gu, with max |dgu| in absmax.
 * [llmq model] LLamaModel::_backward_block: backward_qmm's data gradient
 * through the down projection (dSwiGLU) followed by swiglu_backward(DMlpUp,
 * DSwiGLU, MlpUp, ...); the two calls run as one kernel, so dSwiGLU never
 * reaches memory.  dgu: bf16 [M, 2H] (gate columns, then up columns); gu: bf16
 * [M, 2H], the forward's gate+up output (dgu may be gu: updated in place);
 * a: [M,K], b: [H,K], dtype and scales as ffn_matmul_tn; flags: 0,
 * FFN_TN_TILE_GRID and/or FFN_TN_TILED; absmax: fp32 [1] or NULL.  Supported: K % 128 == 0,
 * H % 128 == 0, any M >= 0; dgu must not alias a or b. */
ffn_status_t ffn_matmul_tn_swiglu_bwd(void* dgu, float* absmax, const void* a,
                                      const float* a_scale, const void* b, const float* b_scale,
                                      const void* gu, ffn_dtype_t dtype, int flags, int64_t M,
                                      int64_t H, int64_t K, hipStream_t stream);

/* ffn_matmul_tn_swiglu_bwd that max-accumulates max|dgu| into *absmax
 * (required) as found instead of clearing it first (the dMlpUp slot of the
 * abs-max table, [llmq model] LLamaRunState: DMlpUp.Quant.Stats); other
 * arguments and checks as ffn_matmul_tn_swiglu_bwd. */
ffn_status_t ffn_matmul_tn_swiglu_bwd_acc(void* dgu, float* absmax, const void* a,
                                          const float* a_scale, const void* b,
                                          const float* b_scale, const void* gu, ffn_dtype_t dtype,
                                          int flags, int64_t M, int64_t H, int64_t K,
                                          hipStream_t stream);

/* Transpose: out[c, r] = in[r, c] for r < rows, and 0 for rows <= r < ld_out
 * (zero padding that rounds a token count up to ffn_matmul_tn's K granularity).
 * [llmq model] backward_qmm, transpose(weight_tp, ...), transpose(activation_tp,
 * ...), transpose(grad_tp, ...).  in: [rows, cols]; out: [cols, ld_out];
 * elt_bytes 2 (bf16) or 1 (e4m3 codes).  Supported: cols % 16 == 0,
 * ld_out % 16 == 0, ld_out >= rows; out must not alias in. */
ffn_status_t ffn_transpose(void* out, const void* in, int64_t rows, int64_t cols,
                           int64_t ld_out, int elt_bytes, hipStream_t stream);

/* Quantise with a known abs-max and transpose in one pass: q_t[c, r] =
 * fp8(x[r, c] * max / absmax), *scale = absmax / max (1 and 1 for absmax 0),
 * zero codes for rows <= r < ld_out; max = 448 for code_dtype FFN_E4M3, 57344
 * for FFN_E5M2 (codes saturate at +-max).  [llmq model] backward_qmm,
 * quantize_and_transpose_with_abs_max into the grad dtype (and, with q,
 * quantize_with_abs_max of the same tensor from the same read: backward_qmm
 * quantises the output gradient in both layouts).  x: bf16 [rows, cols]; q_t:
 * codes [cols, ld_out]; q (nullable): codes [rows, cols] in x's layout;
 * absmax: fp32 [1] (device, read).  Constraints as ffn_transpose; q must not
 * alias q_t or x. */
ffn_status_t ffn_quant_transpose(uint8_t* q_t, uint8_t* q, float* scale, const void* x,
                                 const float* absmax, ffn_dtype_t code_dtype, int64_t rows,
                                 int64_t cols, int64_t ld_out, hipStream_t stream);

/* ffn_quant_transpose that also sets *clear (required; fp32 [1], another
 * word than scale and absmax) to zero: the consumer of one abs-max slot
 * clears the slot of the next producer, so that a backward step needs no
 * clearing launch (ffn_quant_absmax_clear is the forward's counterpart). */
ffn_status_t ffn_quant_transpose_clear(uint8_t* q_t, uint8_t* q, float* scale, const void* x,
                                       const float* absmax, float* clear, ffn_dtype_t code_dtype,
                                       int64_t rows, int64_t cols, int64_t ld_out,
                                       hipStream_t stream);

/* SwiGLU backward.  [llmq model] _backward_block, swiglu_backward(DMlpUp,
 * DSwiGLU, MlpUp, DMlpUp abs-max, B, T, D).  With g = gu[n,j], u = gu[n,H+j],
 * s = 1/(1+exp(-g)):
 *   dgu[n,j]   = bf16(dh[n,j] * u * s * (1 + g * (1 - s)))
 *   dgu[n,H+j] = bf16(dh[n,j] * g * s)
 * dgu: bf16 [N,2H] (may be gu itself: the trainer writes it over MlpUp);
 * dh: bf16 [N,H]; absmax (nullable) receives max |dgu|.  Supported: H % 8 == 0;
 * dgu must not alias dh. */
ffn_status_t ffn_swiglu_bwd(void* dgu, float* absmax, const void* dh, const void* gu,
                            int64_t N, int64_t H, hipStream_t stream);

/* ffn_swiglu_bwd that max-accumulates max|dgu| into *absmax (required) as
 * found; other arguments and checks as ffn_swiglu_bwd. */
ffn_status_t ffn_swiglu_bwd_acc(void* dgu, float* absmax, const void* dh, const void* gu,
                                int64_t N, int64_t H, hipStream_t stream);

/* RMSNorm backward with the saved rstd, added to the residual stream's
 * gradient.  [llmq model] _backward_block, rmsnorm_backward(DResAtt, LN2_w
 * grad, scratch, DResFFN, DLN2, ResidualAtt, LN2_w, LN2_Rstd, DResAtt abs-max,
 * B, T, C).  With xh = r * rstd, gy = dy * w, m = sum_j gy_j xh_j / C:
 *   dinp[n,j]  = bf16(dresidual[n,j] + rstd_n * (gy_j - xh_j * m))
 *   dweight[j] += sum_n dy[n,j] * xh[n,j]      (fp32, fixed summation order)
 * dinp, dresidual, dy, r: bf16 [N,C] (dinp may be dresidual); weight: bf16 [C];
 * rstd: fp32 [N]; dweight: fp32 [C], accumulated; absmax (nullable) receives
 * max |dinp|; scratch: device memory of ffn_rmsnorm_bwd_scratch_bytes(N, C)
 * bytes (the per-wave partial weight gradients; its size is not checked).
 * Supported: C % 8 == 0, C <= 8192. */
int64_t ffn_rmsnorm_bwd_scratch_bytes(int64_t N, int64_t C);
ffn_status_t ffn_rmsnorm_bwd(void* dinp, float* dweight, float* scratch,
                             const void* dresidual, const void* dy, const void* r,
                             const void* weight, const float* rstd, float* absmax,
                             int64_t N, int64_t C, hipStream_t stream);

/* ffn_rmsnorm_bwd that max-accumulates max|dinp| into *absmax (required; the
 * DResAtt slot) as found, and sets *clear (nullable; another word than
 * absmax) to zero: the slot whose consumer ran before this pass (dMlpUp's,
 * read by ffn_quant_transpose_clear), ready for the next step's producer.
 * Other arguments and checks as ffn_rmsnorm_bwd. */
ffn_status_t ffn_rmsnorm_bwd_acc(void* dinp, float* dweight, float* scratch,
                                 const void* dresidual, const void* dy, const void* r,
                                 const void* weight, const float* rstd, float* absmax,
                                 float* clear, int64_t N, int64_t C, hipStream_t stream);

/* Thread-local text for the last non-OK status of this thread ("" if none). */
/* The backward's FP8 products on tiled operands (the layout of the tiled
 * prefill entry points, with whole 64-row groups).  FFN_TN_TILED in the
 * flags of ffn_matmul_tn, ffn_matmul_tn_swiglu_bwd and
 * ffn_matmul_tn_swiglu_bwd_acc: a [M, K] and b [N, K] (codes) are tiled, the
 * outputs stay row-major; the results equal the row-major call's bit for
 * bit.  ffn_transpose_tiled: ffn_transpose of e4m3 codes (1-byte elements)
 * with out [cols, ld_out] stored tiled (ffn_tile_bytes(cols, ld_out) bytes).
 * ffn_quant_transpose_tiled: ffn_quant_transpose with q_t [cols, ld_out] and
 * q [rows, cols] (if given) stored tiled and clear (nullable) zeroed as in
 * ffn_quant_transpose_clear.  Both need cols % 64 == 0 and ld_out % 64 ==
 * 0; the rows past cols (q_t) or rows (q) in the last group are not
 * written.  [llmq model] LLamaModel::_backward_block, backward_qmm. */
ffn_status_t ffn_transpose_tiled(uint8_t* out, const uint8_t* in, int64_t rows, int64_t cols,
                                 int64_t ld_out, hipStream_t stream);
ffn_status_t ffn_quant_transpose_tiled(uint8_t* q_t, uint8_t* q, float* scale, const void* x,
                                       const float* absmax, float* clear, ffn_dtype_t code_dtype,
                                       int64_t rows, int64_t cols, int64_t ld_out, hipStream_t stream);

const char* ffn_last_error(void);

/* Library version string. */
const char* ffn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFN_H */
