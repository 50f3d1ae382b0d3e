// Host-side launchers of the FFN kernels (internal to libffn.so).  Each returns
// the HIP status of its launches; arguments are validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

hipError_t launch_fill(float* p, int n, float v, hipStream_t s);
// compute units of the current device (cached per device; 256 if unknown)
int device_cu_count();
// clear_absmax == false: *absmax is max-accumulated into as found (the
// caller zeroed it), not cleared first.  tiled_y: y in the tiled GEMM
// operand layout of [N, 2C bytes] (common.h, tiled_offset).
hipError_t launch_rmsnorm(uint16_t* y, float* rstd, uint16_t* res, float* absmax, const uint16_t* inp,
                          const uint16_t* add, const uint16_t* w, float eps, int64_t N, int C, hipStream_t s,
                          bool clear_absmax = true, bool tiled_y = false);
hipError_t launch_absmax(float* absmax, const uint16_t* x, int64_t n, hipStream_t s);
// clear (nullable): another abs-max word that the kernel sets to zero.
hipError_t launch_quant(uint8_t* q, float* scale, float* absmax, const uint16_t* x, int64_t n, bool compute,
                        hipStream_t s, float* clear = nullptr);
hipError_t launch_quant_rows(uint8_t* q, float* row_scale, const uint16_t* w, int64_t rows, int cols,
                             hipStream_t s);
hipError_t launch_swiglu(uint16_t* h, float* absmax, const uint16_t* gu, int64_t N, int H, hipStream_t s);

// GEMM: out[n, o] = sum_k x[n, k] * w[o, k] (optionally scaled, optionally
// SwiGLU-fused).  fp8 selects e4m3 operands with device scales.
// q_absmax / q_scale: SwiGLU only; out then holds e4m3 codes of h quantised
// with the known abs-max *q_absmax, and *q_scale receives its scale.
// accumulate (plain output only): out = bf16(out + product), one rounding.
// x_e5m2 (fp8, plain output only): x holds e5m2 codes (w stays e4m3).
// swiglu_gu (plain output, no accumulation): the product is dh = dL/dh of
// h = silu(g) * u, rounded to bf16; out receives dgu [N, 2O] computed from
// gu [N, 2O] (which out may be), and absmax max |dgu|.  tile_grid: one
// workgroup per output tile (for products that run beside others).  tiled:
// x and w in the tiled layout (whole 64-row groups; common.h, tiled_offset),
// with every epilogue for FP8 operands and the SwiGLU and plain ones for
// bf16; the SwiGLU output is stored in it too when it is a GEMM operand
// itself (the e4m3 codes of q_absmax, or bf16 h of a bf16 product),
// row-major otherwise (bf16 h of an e4m3 product, which a quantiser reads;
// the products and gradients of the plain, accumulating and SwiGLU-backward
// epilogues).
hipError_t launch_gemm(void* out, float* absmax, const void* x, const float* x_scale, const void* w,
                       const float* w_scale, bool fp8, bool fuse_swiglu, int64_t N, int K, int O,
                       hipStream_t s, const float* q_absmax = nullptr, float* q_scale = nullptr,
                       bool accumulate = false, bool x_e5m2 = false, const void* swiglu_gu = nullptr,
                       bool tile_grid = false, bool clear_absmax = true, bool tiled = false);
// The tiled layout of a [rows, row_bytes] operand (row_bytes % 64 == 0), in
// whole 64-row groups: rows past `rows` in the last group are zero.
hipError_t launch_tile_pack(uint8_t* out, const uint8_t* in, int64_t rows, int64_t row_bytes, hipStream_t s);
// launch_quant with the codes of x [rows, cols] stored in the tiled layout
// (cols % 64 == 0; rows past `rows` in the last group are left as they are).
hipError_t launch_quant_tiled(uint8_t* q, float* scale, float* absmax, const uint16_t* x, int64_t rows, int64_t cols,
                              hipStream_t s, float* clear = nullptr);

// Backward: out[c, r] = in[r, c], zero for rows <= r < ld_out.  (in_bytes,
// out_bytes) = (2, 2) bf16, (1, 1) e4m3 codes, (2, 1) bf16 quantised to e4m3
// with *absmax on the way (scale written to *scale; q_rows, if not null, also
// receives the codes in the input's [rows, cols] layout; e5m2: e5m2 codes;
// clear, if not null, another abs-max word that the quantising pass zeroes;
// tiled_out (byte outputs only): out and q_rows in the tiled GEMM operand
// layout, rows of ld_out and cols bytes).
hipError_t launch_transpose(void* out, uint8_t* q_rows, float* scale, const float* absmax, const void* in,
                            int64_t rows, int cols, int64_t ld_out, int in_bytes, int out_bytes, hipStream_t s,
                            bool e5m2 = false, float* clear = nullptr, bool tiled_out = false);
// clear_absmax == false: *absmax is max-accumulated into as found.
hipError_t launch_swiglu_bwd(uint16_t* dgu, float* absmax, const uint16_t* dh, const uint16_t* gu, int64_t N, int H,
                             hipStream_t s, bool clear_absmax = true);
// scratch: rmsnorm_bwd_scratch_floats(N, C) floats.  clear_absmax == false:
// *absmax is max-accumulated into as found; clear (nullable): another abs-max
// word that the pass zeroes.
int64_t rmsnorm_bwd_scratch_floats(int64_t N, int C);
hipError_t launch_rmsnorm_bwd(uint16_t* dinp, float* dweight, float* scratch, const uint16_t* dres,
                              const uint16_t* dy, const uint16_t* r, const uint16_t* w, const float* rstd,
                              float* absmax, int64_t N, int C, hipStream_t s, bool clear_absmax = true,
                              float* clear = nullptr);

// Decode arms (the caller has checked: arms other than the split one, and bf16
// weights, only for M <= 4; gu is a [M, 2H] bf16 workspace for those arms).
enum : int { kDecodeSplitSilu = 0, kDecodeSiluInput = 1, kDecodePerProjection = 2 };
hipError_t launch_decode(uint16_t* out, uint16_t* h, uint16_t* gu, const uint16_t* x, const uint8_t* wg,
                         const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd, const float* sd,
                         int arm, bool bf16_weights, int M, int C, int H, hipStream_t s);
// Packed decode: launch_pack_weight writes the packed layout of an e4m3
// [rows, cols] weight (rows % 16 == 0, cols % 64 == 0); launch_decode_packed
// runs the split-SiLU decode on packed weights for 1 <= M <= 32 with ws
// (decode_packed_ws_elems(M, C, H) bf16 elements) for the fragment-order
// copies of x and h.
hipError_t launch_pack_weight(uint8_t* dst, const uint8_t* w, int64_t rows, int cols, hipStream_t s);
int64_t decode_packed_ws_elems(int M, int C, int H);
hipError_t launch_decode_packed(uint16_t* out, uint16_t* h, uint16_t* ws, const uint16_t* x, const uint8_t* wg,
                                const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd,
                                const float* sd, int M, int C, int H, hipStream_t s);

}  // namespace ffn
