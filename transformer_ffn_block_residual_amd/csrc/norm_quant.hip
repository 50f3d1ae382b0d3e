// Bandwidth-bound kernels of the FFN block: fused residual add + RMSNorm with
// rstd and abs-max, abs-max reduction, e4m3 quantisation (per tensor and per
// row) and the standalone SwiGLU.
//
// Every kernel reads and writes HBM in 16-byte vectors per lane, consecutive
// lanes on consecutive addresses, and folds its abs-max into the same pass
// (one atomic per workgroup on the bit pattern of a non-negative float).
#include "common.h"
#include "launch.h"

namespace ffn {

// ---------------------------------------------------------------------------
// Fill: clears abs-max slots.  A kernel rather than hipMemsetAsync so that a
// captured graph replays it reliably.
__global__ void fill_f32_kernel(float* p, int n, float v) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill(float* p, int n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((n + 63) / 64), dim3(64), 0, s, p, n, v);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused residual add + RMSNorm (llmq llama_model.cpp, LLamaModel::_forward_block,
// fused_residual_rmsnorm_forward).  One wave per row; the row stays in
// registers (CPL 16-byte chunks per lane), so y may overwrite inp or addend.
//   r = bf16(inp + addend); rstd = 1/sqrt(sum r^2 / C + eps);
//   y = bf16((r * rstd) * w); absmax = max |y|.
// kTiledY: y is stored in the tiled GEMM operand layout of [N, 2C bytes]
// (common.h, tiled_offset; each 16-byte chunk stays whole), for a bf16
// gate+up projection on tiled operands.
template <int CPL, bool kAdd, bool kTiledY>
__global__ __launch_bounds__(256) void rmsnorm_kernel(
    uint16_t* y, float* rstd_out, uint16_t* res_out, float* absmax,
    const uint16_t* inp, const uint16_t* addend, const uint16_t* w,
    float eps, int64_t N, int C) {
    __shared__ float red[4];
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nch = C >> 3;  // 8 bf16 per 16-byte chunk
    float amax = 0.0f;
    if (row < N) {
        const uint4* a4 = reinterpret_cast<const uint4*>(inp + row * C);
        const uint4* b4 = reinterpret_cast<const uint4*>(addend + row * C);
        // All loads are issued before any use: chunks past the row end load
        // the row's last chunk again (in bounds, no branch that would make the
        // compiler wait after every load) and are left out of the sum.
        // The longest rows add the addend in groups of 8 chunks as well.
        constexpr bool kGroupAdd = kAdd && CPL > 16;
        uint4 r[CPL], bv[kGroupAdd ? 1 : CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = min(lane + i * 64, nch - 1);
            r[i] = a4[c];
            if (kAdd && !kGroupAdd) bv[i] = b4[c];
        }
        if (kGroupAdd) {
#pragma unroll
            for (int i0 = 0; i0 < CPL; i0 += 8) {
                __builtin_amdgcn_sched_barrier(0);
                uint4 bg[8];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) bg[ii] = b4[min(lane + (i0 + ii) * 64, nch - 1)];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    uint32_t* ap = reinterpret_cast<uint32_t*>(&r[i0 + ii]);
                    const uint32_t* bp = reinterpret_cast<const uint32_t*>(&bg[ii]);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        ap[q] = pack_bf16x2(bf16lo(ap[q]) + bf16lo(bp[q]), bf16hi(ap[q]) + bf16hi(bp[q]));
                }
            }
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            if (kAdd && !kGroupAdd) {
                uint32_t* ap = reinterpret_cast<uint32_t*>(&r[i]);
                const uint32_t* bp = reinterpret_cast<const uint32_t*>(&bv[i]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    ap[q] = pack_bf16x2(bf16lo(ap[q]) + bf16lo(bp[q]), bf16hi(ap[q]) + bf16hi(bp[q]));
            }
            const uint32_t* rp = reinterpret_cast<const uint32_t*>(&r[i]);
            float part = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float lo = bf16lo(rp[q]), hi = bf16hi(rp[q]);
                part += lo * lo;
                part += hi * hi;
            }
            ss += lane + i * 64 < nch ? part : 0.0f;
        }
        if (CPL > 16) {
            // the longest rows: keep the row packed between the two passes
            // (the compiler would otherwise hold its unpacked fp32 copy too)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                uint32_t* rp = reinterpret_cast<uint32_t*>(&r[i]);
                asm volatile("" : "+v"(rp[0]), "+v"(rp[1]), "+v"(rp[2]), "+v"(rp[3]));
            }
        }
        ss = wave_sum(ss);
        const float rs = 1.0f / sqrtf(ss / (float)C + eps);
        if (lane == 0) rstd_out[row] = rs;
        const uint4* w4 = reinterpret_cast<const uint4*>(w);
        uint4* y4 = reinterpret_cast<uint4*>(y + row * C);
        uint4* o4 = kAdd ? reinterpret_cast<uint4*>(res_out + row * C) : nullptr;
        // the longest rows (32 chunks per lane) take their weights in groups of
        // 8 chunks, so that the row and its weights never fill the registers
        constexpr int kWG = CPL > 16 ? 8 : CPL;
#pragma unroll
        for (int i0 = 0; i0 < CPL; i0 += kWG) {
            // (a group's loads are not hoisted above the previous group's use)
            if (kWG < CPL) __builtin_amdgcn_sched_barrier(0);
            uint4 wr[kWG];
#pragma unroll
            for (int i = 0; i < kWG; ++i) wr[i] = w4[min(lane + (i0 + i) * 64, nch - 1)];
#pragma unroll
            for (int ii = 0; ii < kWG; ++ii) {
                const int i = i0 + ii;
                const int c = lane + i * 64;
                if (c < nch) {
                    const uint4 wv = wr[ii];
                    const uint32_t* rp = reinterpret_cast<const uint32_t*>(&r[i]);
                    const uint32_t* wp = reinterpret_cast<const uint32_t*>(&wv);
                    uint4 yv;
                    uint32_t* yp = reinterpret_cast<uint32_t*>(&yv);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        yp[q] = pack_bf16x2((bf16lo(rp[q]) * rs) * bf16lo(wp[q]),
                                            (bf16hi(rp[q]) * rs) * bf16hi(wp[q]));
                        amax = absmax_acc(absmax_acc(amax, bf16lo(yp[q])), bf16hi(yp[q]));
                    }
                    if (kAdd) o4[c] = r[i];
                    if (kTiledY)
                        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(y) +
                                                  tiled_offset(row, (int64_t)c * 16, 2 * (int64_t)C)) = yv;
                    else
                        y4[c] = yv;
                }
            }
        }
    }
    if (absmax) block_absmax_commit(amax, red, absmax);
}

template <int CPL, bool kTiledY>
static void launch_rmsnorm_cpl(uint16_t* y, float* rstd, uint16_t* res, float* absmax, const uint16_t* inp,
                               const uint16_t* add, const uint16_t* w, float eps, int64_t N, int C,
                               hipStream_t s) {
    dim3 grid((unsigned)((N + 3) / 4)), block(256);
    if (add)
        hipLaunchKernelGGL((rmsnorm_kernel<CPL, true, kTiledY>), grid, block, 0, s, y, rstd, res, absmax, inp, add, w,
                           eps, N, C);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<CPL, false, kTiledY>), grid, block, 0, s, y, rstd, res, absmax, inp, add, w,
                           eps, N, C);
}

template <bool kTiledY>
static void launch_rmsnorm_any(uint16_t* y, float* rstd, uint16_t* res, float* absmax, const uint16_t* inp,
                               const uint16_t* add, const uint16_t* w, float eps, int64_t N, int C,
                               hipStream_t s) {
    const int need = (C / 8 + 63) / 64;  // chunks per lane
    if (need <= 1) launch_rmsnorm_cpl<1, kTiledY>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    else if (need <= 2) launch_rmsnorm_cpl<2, kTiledY>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    else if (need <= 4) launch_rmsnorm_cpl<4, kTiledY>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    else if (need <= 8) launch_rmsnorm_cpl<8, kTiledY>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    else if (need <= 16) launch_rmsnorm_cpl<16, kTiledY>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    else launch_rmsnorm_cpl<32, kTiledY>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
}

hipError_t launch_rmsnorm(uint16_t* y, float* rstd, uint16_t* res, float* absmax, const uint16_t* inp,
                          const uint16_t* add, const uint16_t* w, float eps, int64_t N, int C, hipStream_t s,
                          bool clear_absmax, bool tiled_y) {
    if (absmax && clear_absmax) {
        hipError_t e = launch_fill(absmax, 1, 0.0f, s);
        if (e != hipSuccess) return e;
    }
    if (N == 0) return hipSuccess;
    if (tiled_y) launch_rmsnorm_any<true>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    else launch_rmsnorm_any<false>(y, rstd, res, absmax, inp, add, w, eps, N, C, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Standalone abs-max of a bf16 tensor (llmq llama_model.cpp, _forward_block,
// abs_max).  Grid-stride over groups of four 16-byte chunks per thread (four
// loads in flight before any is used); any length (scalar tail).
__global__ __launch_bounds__(256) void absmax_kernel(float* out, const uint16_t* __restrict__ x, int64_t n) {
    __shared__ float red[4];
    float m = 0.0f;
    const int64_t nch = n >> 3;
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t c = t0; c < nch; c += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t ci = c + i * stride;
            v[i] = ci < nch ? x4[ci] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(&v[i]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                m = absmax_acc(absmax_acc(m, bf16lo(p[q])), bf16hi(p[q]));
        }
    }
    for (int64_t i = (nch << 3) + t0; i < n; i += stride) m = absmax_acc(m, bf16lo(x[i]));
    block_absmax_commit(m, red, out);
}

// ---------------------------------------------------------------------------
// Per-tensor e4m3 quantisation with a known abs-max (llmq llama_model.cpp,
// forward_qmm, quantize_with_abs_max).  16 elements per thread: two 16-byte
// loads, one 16-byte store.  inv = 448/absmax in IEEE fp32; codes from the fp32
// product x*inv.  Block 0 also writes the scale absmax/448 and, when given,
// zero to *clear (another tensor's abs-max word, for its next producer).

// 16 bf16 values (v0: the first 8) -> their 16 e4m3 codes of x * inv.
__device__ __forceinline__ uint4 quant16(const uint4 v0, const uint4 v1, float inv) {
    uint4 o;
    o.x = pack_e4m3x4(bf16lo(v0.x) * inv, bf16hi(v0.x) * inv, bf16lo(v0.y) * inv, bf16hi(v0.y) * inv);
    o.y = pack_e4m3x4(bf16lo(v0.z) * inv, bf16hi(v0.z) * inv, bf16lo(v0.w) * inv, bf16hi(v0.w) * inv);
    o.z = pack_e4m3x4(bf16lo(v1.x) * inv, bf16hi(v1.x) * inv, bf16lo(v1.y) * inv, bf16hi(v1.y) * inv);
    o.w = pack_e4m3x4(bf16lo(v1.z) * inv, bf16hi(v1.z) * inv, bf16lo(v1.w) * inv, bf16hi(v1.w) * inv);
    return o;
}

__global__ __launch_bounds__(256) void quant_kernel(uint8_t* __restrict__ q, float* __restrict__ scale_out,
                                                    const float* __restrict__ absmax,
                                                    const uint16_t* __restrict__ x, int64_t n,
                                                    float* __restrict__ clear) {
    float scale, inv;
    scale_pair(*absmax, scale, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *scale_out = scale;
        if (clear) *clear = 0.0f;
    }
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t base = t * 16;
    if (base + 16 <= n) {
        const uint4* x4 = reinterpret_cast<const uint4*>(x + base);
        *reinterpret_cast<uint4*>(q + base) = quant16(x4[0], x4[1], inv);
    } else if (base < n) {
        for (int64_t i = base; i < n; ++i) {
            const float v = bf16lo(x[i]) * inv;
            q[i] = (uint8_t)(pack_e4m3x4(v, 0.0f, 0.0f, 0.0f) & 0xff);
        }
    }
}

// The same codes stored in the tiled GEMM operand layout of [rows, cols]
// (common.h, tiled_offset; cols % 64 == 0, rows * cols / 16 < 2^32).  In
// that layout the 64 codes of K-step s of rows 2m and 2m + 1 share one
// 128-byte line, so a wave takes such a row pair over 8 K-steps: lane l
// quantises the 16 elements of chunk l % 4 of K-step (l / 4) % 8 of row
// 2m + l / 32.  Each wave reads 1 KiB of each of its two rows and stores
// eight whole lines.  Rows past `rows` are not written.
__global__ __launch_bounds__(256) void quant_tiled_kernel(uint8_t* __restrict__ q, float* __restrict__ scale_out,
                                                          const float* __restrict__ absmax,
                                                          const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, float* __restrict__ clear) {
    float scale, inv;
    scale_pair(*absmax, scale, inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *scale_out = scale;
        if (clear) *clear = 0.0f;
    }
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t wv = t >> 6, l = t & 63;
    const uint32_t steps = (uint32_t)(cols >> 6), runs = (steps + 7) / 8;
    const uint32_t pair = wv / runs, run = wv - pair * runs;
    const int64_t r = 2 * (int64_t)pair + (l >> 5);
    const uint32_t s = run * 8 + ((l >> 2) & 7);
    if (r >= rows || s >= steps) return;
    const int64_t c = 64 * (int64_t)s + 16 * (l & 3);
    const uint4* x4 = reinterpret_cast<const uint4*>(x + r * cols + c);
    *reinterpret_cast<uint4*>(q + tiled_offset(r, c, cols)) = quant16(x4[0], x4[1], inv);
}

hipError_t launch_quant_tiled(uint8_t* q, float* scale, float* absmax, const uint16_t* x, int64_t rows, int64_t cols,
                              hipStream_t s, float* clear) {
    const int64_t waves = (rows + 1) / 2 * (((cols >> 6) + 7) / 8);
    const int64_t blocks = waves > 0 ? (waves + 3) / 4 : 1;  // no rows: still writes the scale
    hipLaunchKernelGGL(quant_tiled_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, scale, absmax, x, rows, cols,
                       clear);
    return hipGetLastError();
}

hipError_t launch_absmax(float* absmax, const uint16_t* x, int64_t n, hipStream_t s) {
    hipError_t e = launch_fill(absmax, 1, 0.0f, s);
    if (e != hipSuccess || n == 0) return e;
    int64_t nch = (n + 7) / 8;
    int64_t blocks = (nch + 1023) / 1024;  // four chunks per thread per pass
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, absmax, x, n);
    return hipGetLastError();
}

hipError_t launch_quant(uint8_t* q, float* scale, float* absmax, const uint16_t* x, int64_t n, bool compute,
                        hipStream_t s, float* clear) {
    if (compute) {
        hipError_t e = launch_absmax(absmax, x, n, s);
        if (e != hipSuccess) return e;
    }
    const int64_t threads = (n + 15) / 16;
    const int64_t blocks = threads > 0 ? (threads + 255) / 256 : 1;  // n == 0 still writes the scale
    hipLaunchKernelGGL(quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, scale, absmax, x, n, clear);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row e4m3 quantisation of a weight matrix (the row_scale layout of the FP8
// decode weights, metrale dense_ffn_decode.rs, DenseFfnLayer::forward).  One
// workgroup per row: pass 1 finds the row's abs-max, pass 2 (re-reading the row
// from cache) writes the codes.  cols % 8 == 0.
__global__ __launch_bounds__(256) void quant_rows_kernel(uint8_t* __restrict__ q, float* __restrict__ row_scale,
                                                         const uint16_t* __restrict__ w, int cols) {
    __shared__ float red[4];
    __shared__ float am_s;
    const int64_t row = blockIdx.x;
    const uint4* w4 = reinterpret_cast<const uint4*>(w + row * cols);
    const int nch = cols >> 3;
    float m = 0.0f;
    for (int c = threadIdx.x; c < nch; c += 256) {
        const uint4 v = w4[c];
        const uint32_t* p = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m = absmax_acc(absmax_acc(m, bf16lo(p[k])), bf16hi(p[k]));
    }
    m = wave_absmax(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) am_s = absmax_acc(absmax_acc(red[0], red[1]), absmax_acc(red[2], red[3]));
    __syncthreads();
    float scale, inv;
    scale_pair(am_s, scale, inv);
    if (threadIdx.x == 0) row_scale[row] = scale;
    uint2* q2 = reinterpret_cast<uint2*>(q + row * cols);
    for (int c = threadIdx.x; c < nch; c += 256) {
        const uint4 v = w4[c];
        const uint32_t* p = reinterpret_cast<const uint32_t*>(&v);
        uint2 o;
        o.x = pack_e4m3x4(bf16lo(p[0]) * inv, bf16hi(p[0]) * inv, bf16lo(p[1]) * inv, bf16hi(p[1]) * inv);
        o.y = pack_e4m3x4(bf16lo(p[2]) * inv, bf16hi(p[2]) * inv, bf16lo(p[3]) * inv, bf16hi(p[3]) * inv);
        q2[c] = o;
    }
}

hipError_t launch_quant_rows(uint8_t* q, float* row_scale, const uint16_t* w, int64_t rows, int cols,
                             hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)rows), dim3(256), 0, s, q, row_scale, w, cols);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Standalone SwiGLU (llmq llama_model.cpp, _forward_block, swiglu_forward):
// h[n,j] = bf16(silu(g) * u), g = gu[n,j], u = gu[n,H+j], plus max|h|.
// 8 outputs per thread: one 16-byte load from each half, one 16-byte store.
__global__ __launch_bounds__(256) void swiglu_kernel(uint16_t* __restrict__ h, float* absmax,
                                                     const uint16_t* __restrict__ gu, int64_t N, int H) {
    __shared__ float red[4];
    const int hch = H >> 3;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    float m = 0.0f;
    if (t < N * hch) {
        const int64_t n = t / hch;
        const int c = (int)(t - n * hch);
        const uint4 gv = reinterpret_cast<const uint4*>(gu + n * 2 * H)[c];
        const uint4 uv = reinterpret_cast<const uint4*>(gu + n * 2 * H + H)[c];
        const uint32_t* gp = reinterpret_cast<const uint32_t*>(&gv);
        const uint32_t* up = reinterpret_cast<const uint32_t*>(&uv);
        uint4 o;
        uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            op[k] = pack_bf16x2(silu_mul(bf16lo(gp[k]), bf16lo(up[k])), silu_mul(bf16hi(gp[k]), bf16hi(up[k])));
            m = absmax_acc(absmax_acc(m, bf16lo(op[k])), bf16hi(op[k]));
        }
        reinterpret_cast<uint4*>(h + n * H)[c] = o;
    }
    if (absmax) block_absmax_commit(m, red, absmax);
}

hipError_t launch_swiglu(uint16_t* h, float* absmax, const uint16_t* gu, int64_t N, int H, hipStream_t s) {
    if (absmax) {
        hipError_t e = launch_fill(absmax, 1, 0.0f, s);
        if (e != hipSuccess) return e;
    }
    if (N == 0) return hipSuccess;
    const int64_t threads = N * (H / 8);
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, h, absmax, gu, N, H);
    return hipGetLastError();
}

}  // namespace ffn
