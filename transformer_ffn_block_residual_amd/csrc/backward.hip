// The FFN block's backward kernels (llmq llama_model.cpp,
// LLamaModel::_backward_block and backward_qmm): transposes (with an optional
// e4m3 quantisation on the way) that put the backward products' operands in
// the K-contiguous layout of the MFMA GEMM, the SwiGLU backward and the
// RMSNorm backward.  All are HBM-bound; none allocates.

#include "common.h"
#include "launch.h"

namespace ffn {

// ---------------------------------------------------------------------------
// Transpose: out[c, r] = in[r, c] for r < rows, zero for rows <= r < ld_out
// (the padding that rounds a token count up to the GEMM's K granularity).
// kIn / kOut: element bytes of input and output (2, 2: bf16; 1, 1: e4m3
// codes; 2, 1 with kQuant: e4m3(x * inv), the codes quantize_with_abs_max
// gives, in the transposed layout, and with q_rows also in the input's
// layout, from the same read).  A workgroup moves one 64 x 64 tile
// through LDS: 16-byte loads along input rows, 16-byte stores along output
// rows.  The LDS row pitch is an odd number of dwords so that the column
// gathers spread over the banks.
// (Used for bf16; the byte-output forms use transpose8_kernel below.)
template <int kIn, int kOut, bool kQuant>
__global__ __launch_bounds__(256) void transpose_kernel(uint8_t* __restrict__ out, uint8_t* __restrict__ q_rows,
                                                        float* __restrict__ scale_out,
                                                        const float* __restrict__ absmax,
                                                        const uint8_t* __restrict__ in, int64_t rows, int cols,
                                                        int64_t ld_out) {
    constexpr int kT = 64;                        // tile edge (elements)
    constexpr int kPitch = kT * kOut + 4;         // LDS bytes per tile row
    constexpr int kInEl = 16 / kIn;               // input elements per 16-byte chunk
    constexpr int kOutEl = 16 / kOut;             // output elements per 16-byte chunk
    constexpr int kInCpr = kT / kInEl;            // input chunks per tile row
    constexpr int kOutCpr = kT / kOutEl;          // output chunks per output tile row
    __shared__ __attribute__((aligned(16))) uint8_t tile[kT * kPitch];
    const int c0 = blockIdx.x * kT;
    const int64_t r0 = (int64_t)blockIdx.y * kT;
    float inv = 1.0f;
    if (kQuant) {
        float scale;
        scale_pair(*absmax, scale, inv);
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *scale_out = scale;
    }
    // all loads first, then the LDS writes
    uint4 v[kT * kInCpr / 256];
#pragma unroll
    for (int i = 0; i < kT * kInCpr / 256; ++i) {
        const int k = threadIdx.x + 256 * i;
        const int row = k / kInCpr, cc = k % kInCpr;
        const int64_t gr = r0 + row;
        const int gc = c0 + cc * kInEl;
        v[i] = (gr < rows && gc < cols) ? *reinterpret_cast<const uint4*>(in + (gr * cols + gc) * kIn)
                                        : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kT * kInCpr / 256; ++i) {
        const int k = threadIdx.x + 256 * i;
        const int row = k / kInCpr, cc = k % kInCpr;
        uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * kPitch + cc * kInEl * kOut);
        if (kQuant) {
            const uint32_t q0 = pack_e4m3x4(bf16lo(v[i].x) * inv, bf16hi(v[i].x) * inv, bf16lo(v[i].y) * inv,
                                            bf16hi(v[i].y) * inv);
            const uint32_t q1 = pack_e4m3x4(bf16lo(v[i].z) * inv, bf16hi(v[i].z) * inv, bf16lo(v[i].w) * inv,
                                            bf16hi(v[i].w) * inv);
            dst[0] = q0;
            dst[1] = q1;
            const int64_t gr = r0 + row;
            const int gc = c0 + cc * kInEl;
            if (q_rows && gr < rows && gc < cols)
                *reinterpret_cast<uint2*>(q_rows + gr * cols + gc) = make_uint2(q0, q1);
        } else {
            dst[0] = v[i].x;
            dst[1] = v[i].y;
            dst[2] = v[i].z;
            dst[3] = v[i].w;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kT * kOutCpr / 256; ++i) {
        const int k = threadIdx.x + 256 * i;
        const int c = k / kOutCpr, rc = k % kOutCpr;
        const int go_row = c0 + c;
        const int64_t go_col = r0 + rc * kOutEl;
        uint32_t w[4];
        if (kOut == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = *reinterpret_cast<const uint16_t*>(tile + (rc * 8 + 2 * e) * kPitch + c * 2);
                const uint32_t hi = *reinterpret_cast<const uint16_t*>(tile + (rc * 8 + 2 * e + 1) * kPitch + c * 2);
                w[e] = lo | (hi << 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t x = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) x |= (uint32_t)tile[(rc * 16 + 4 * e + b) * kPitch + c] << (8 * b);
                w[e] = x;
            }
        }
        if (go_row < cols && go_col < ld_out)
            *reinterpret_cast<uint4*>(out + ((int64_t)go_row * ld_out + go_col) * kOut) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Byte-output form (e4m3 codes, plain or quantised on the way): a workgroup
// moves a 128 x 128 tile.  The store side reads LDS a dword at a time (four
// columns of one row) and transposes 4 x 4 byte blocks in registers, so each
// thread writes four 16-byte output chunks (four columns, 16 rows) from 16
// LDS reads, instead of one 16-byte chunk from 16 single-byte reads.  Eight
// consecutive lanes hold the eight 16-row groups of the same four columns, so
// each store instruction writes whole 128-byte lines of eight output rows; the
// row pitch (35 dwords) spreads those lanes' LDS reads over four bank groups.
// kBf8: the quantised codes are e5m2 (scale absmax / 57344) instead of e4m3.
// clear (quantising only, nullable): another abs-max word, set to zero by the
// first thread (the zero-once convention: the word of the next producer).
// kTiledOut: out and q_rows are stored in the tiled GEMM operand layout
// (common.h, tiled_offset; rows of ld_out and cols bytes); every store stays
// one piece of an aligned 16-byte chunk.
template <int kIn, bool kQuant, bool kBf8 = false, bool kTiledOut = false>
__global__ __launch_bounds__(256) void transpose8_kernel(uint8_t* __restrict__ out, uint8_t* __restrict__ q_rows,
                                                         float* __restrict__ scale_out,
                                                         const float* __restrict__ absmax,
                                                         const uint8_t* __restrict__ in, int64_t rows, int cols,
                                                         int64_t ld_out, float* __restrict__ clear) {
    constexpr int kT = 128;                   // tile edge (elements)
    constexpr int kPitch = kT + 12;           // LDS bytes per tile row (35 dwords)
    constexpr int kInEl = 16 / kIn;           // input elements per 16-byte chunk
    constexpr int kInCpr = kT / kInEl;        // input chunks per tile row
    constexpr int kLoads = kT * kInCpr / 256; // input chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t tile[kT * kPitch];
    const int c0 = blockIdx.x * kT;
    const int64_t r0 = (int64_t)blockIdx.y * kT;
    float inv = 1.0f;
    if (kQuant) {
        float scale;
        scale_pair(*absmax, scale, inv, kBf8 ? kE5M2Max : kE4M3Max);
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
            *scale_out = scale;
            if (clear) *clear = 0.0f;
        }
    }
    auto pack4 = [](float a, float b, float c, float d) {
        return kBf8 ? pack_e5m2x4(a, b, c, d) : pack_e4m3x4(a, b, c, d);
    };
    uint4 v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int k = threadIdx.x + 256 * i;
        const int row = k / kInCpr, cc = k % kInCpr;
        const int64_t gr = r0 + row;
        const int gc = c0 + cc * kInEl;
        v[i] = (gr < rows && gc < cols) ? *reinterpret_cast<const uint4*>(in + (gr * cols + gc) * kIn)
                                        : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int k = threadIdx.x + 256 * i;
        const int row = k / kInCpr, cc = k % kInCpr;
        uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * kPitch + cc * kInEl);  // 4-byte aligned
        if (kQuant) {
            const uint32_t q0 = pack4(bf16lo(v[i].x) * inv, bf16hi(v[i].x) * inv, bf16lo(v[i].y) * inv,
                                      bf16hi(v[i].y) * inv);
            const uint32_t q1 = pack4(bf16lo(v[i].z) * inv, bf16hi(v[i].z) * inv, bf16lo(v[i].w) * inv,
                                      bf16hi(v[i].w) * inv);
            dst[0] = q0;
            dst[1] = q1;
            const int64_t gr = r0 + row;
            const int gc = c0 + cc * kInEl;
            if (q_rows && gr < rows && gc < cols)
                *reinterpret_cast<uint2*>(q_rows + (kTiledOut ? tiled_offset(gr, gc, cols) : gr * cols + gc)) =
                    make_uint2(q0, q1);
        } else {
            dst[0] = v[i].x;
            dst[1] = v[i].y;
            dst[2] = v[i].z;
            dst[3] = v[i].w;
        }
    }
    __syncthreads();
    const int rg = threadIdx.x & 7;    // rows 16 rg .. 16 rg + 15 of the tile
    const int cg = threadIdx.x >> 3;   // columns 4 cg .. 4 cg + 3 of the tile
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = *reinterpret_cast<const uint32_t*>(tile + (16 * rg + i) * kPitch + 4 * cg);
    const int64_t go_col = r0 + 16 * rg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // byte j of d[4e .. 4e + 3] -> dword e of column 4 cg + j
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = ((d[4 * e] >> (8 * j)) & 0xffu) | (((d[4 * e + 1] >> (8 * j)) & 0xffu) << 8) |
                   (((d[4 * e + 2] >> (8 * j)) & 0xffu) << 16) | (((d[4 * e + 3] >> (8 * j)) & 0xffu) << 24);
        const int go_row = c0 + 4 * cg + j;
        if (go_row < cols && go_col < ld_out)
            *reinterpret_cast<uint4*>(out + (kTiledOut ? tiled_offset(go_row, go_col, ld_out)
                                                       : (int64_t)go_row * ld_out + go_col)) =
                make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// The scale of a quantising transpose with nothing to transpose (one thread).
template <bool kBf8>
__global__ __launch_bounds__(64) void fp8_scale_kernel(float* __restrict__ scale_out, const float* __restrict__ absmax,
                                                       float* __restrict__ clear) {
    if (threadIdx.x == 0) {
        float scale, inv;
        scale_pair(*absmax, scale, inv, kBf8 ? kE5M2Max : kE4M3Max);
        *scale_out = scale;
        if (clear) *clear = 0.0f;
    }
}

template <bool kTiledOut>
static void launch_transpose8(uint8_t* o, uint8_t* q_rows, float* scale, const float* absmax, const uint8_t* x,
                              int64_t rows, int cols, int64_t ld_out, int in_bytes, hipStream_t s, bool e5m2,
                              float* clear) {
    const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((ld_out + 127) / 128)), block(256);
    if (in_bytes == 1)
        hipLaunchKernelGGL((transpose8_kernel<1, false, false, kTiledOut>), grid, block, 0, s, o, nullptr, nullptr,
                           nullptr, x, rows, cols, ld_out, nullptr);
    else if (e5m2)
        hipLaunchKernelGGL((transpose8_kernel<2, true, true, kTiledOut>), grid, block, 0, s, o, q_rows, scale, absmax,
                           x, rows, cols, ld_out, clear);
    else
        hipLaunchKernelGGL((transpose8_kernel<2, true, false, kTiledOut>), grid, block, 0, s, o, q_rows, scale,
                           absmax, x, rows, cols, ld_out, clear);
}

hipError_t launch_transpose(void* out, uint8_t* q_rows, float* scale, const float* absmax, const void* in,
                            int64_t rows, int cols, int64_t ld_out, int in_bytes, int out_bytes, hipStream_t s,
                            bool e5m2, float* clear, bool tiled_out) {
    if (tiled_out && out_bytes != 1) return hipErrorInvalidValue;
    if (cols == 0 || ld_out == 0) {
        // no codes to write; a quantising call still writes its scale (and
        // clears its word)
        if (in_bytes == 2 && out_bytes == 1) {
            if (e5m2) hipLaunchKernelGGL(fp8_scale_kernel<true>, dim3(1), dim3(64), 0, s, scale, absmax, clear);
            else hipLaunchKernelGGL(fp8_scale_kernel<false>, dim3(1), dim3(64), 0, s, scale, absmax, clear);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    uint8_t* o = static_cast<uint8_t*>(out);
    const uint8_t* x = static_cast<const uint8_t*>(in);
    if (in_bytes == 2 && out_bytes == 2) {
        const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((ld_out + 63) / 64)), block(256);
        hipLaunchKernelGGL((transpose_kernel<2, 2, false>), grid, block, 0, s, o, nullptr, nullptr, nullptr, x, rows,
                           cols, ld_out);
    } else if (tiled_out) {
        launch_transpose8<true>(o, q_rows, scale, absmax, x, rows, cols, ld_out, in_bytes, s, e5m2, clear);
    } else {
        launch_transpose8<false>(o, q_rows, scale, absmax, x, rows, cols, ld_out, in_bytes, s, e5m2, clear);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SwiGLU backward (swiglu_backward): from dh [N, H] and the up-projection
// output gu [N, 2H] (gate columns, then up columns),
//   s = 1 / (1 + exp(-g)),  dg = bf16(dh * u * s * (1 + g * (1 - s))),
//   du = bf16(dh * g * s)
// into dgu [N, 2H] in the same layout, with max |dgu|.  Eight elements of h
// per thread (16-byte loads and stores), grid-stride.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(uint16_t* dgu, float* __restrict__ absmax,
                                                         const uint16_t* __restrict__ dh,
                                                         const uint16_t* gu, int64_t N, int H) {
    __shared__ float red[4];
    const int cpr = H >> 3;  // chunks of 8 per row of h
    const int64_t total = N * cpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    float m = 0.0f;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
        const int64_t n = t / cpr;
        const int j = (int)(t - n * cpr) * 8;
        const uint4 d4 = *reinterpret_cast<const uint4*>(dh + n * H + j);
        const uint4 g4 = *reinterpret_cast<const uint4*>(gu + n * 2 * H + j);
        const uint4 u4 = *reinterpret_cast<const uint4*>(gu + n * 2 * H + H + j);
        const uint32_t* dp = reinterpret_cast<const uint32_t*>(&d4);
        const uint32_t* gp = reinterpret_cast<const uint32_t*>(&g4);
        const uint32_t* up = reinterpret_cast<const uint32_t*>(&u4);
        uint4 og, ou;
        uint32_t* ogp = reinterpret_cast<uint32_t*>(&og);
        uint32_t* oup = reinterpret_cast<uint32_t*>(&ou);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float rg[2], ru[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float d = h ? bf16hi(dp[q]) : bf16lo(dp[q]);
                const float g = h ? bf16hi(gp[q]) : bf16lo(gp[q]);
                const float u = h ? bf16hi(up[q]) : bf16lo(up[q]);
                swiglu_bwd_pair(d, g, u, rg[h], ru[h]);
            }
            ogp[q] = pack_bf16x2(rg[0], rg[1]);
            oup[q] = pack_bf16x2(ru[0], ru[1]);
            m = absmax_acc(absmax_acc(m, bf16lo(ogp[q])), bf16hi(ogp[q]));
            m = absmax_acc(absmax_acc(m, bf16lo(oup[q])), bf16hi(oup[q]));
        }
        *reinterpret_cast<uint4*>(dgu + n * 2 * H + j) = og;
        *reinterpret_cast<uint4*>(dgu + n * 2 * H + H + j) = ou;
    }
    if (absmax) block_absmax_commit(m, red, absmax);
}

hipError_t launch_swiglu_bwd(uint16_t* dgu, float* absmax, const uint16_t* dh, const uint16_t* gu, int64_t N, int H,
                             hipStream_t s, bool clear_absmax) {
    if (absmax && clear_absmax) {
        hipError_t e = launch_fill(absmax, 1, 0.0f, s);
        if (e != hipSuccess) return e;
    }
    if (N == 0) return hipSuccess;
    const int64_t total = N * (H / 8);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s, dgu,
                       absmax, dh, gu, N, H);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm backward (rmsnorm_backward), with the saved rstd:
//   xh = r * rstd,  gy = dy * w,  m = sum_j gy_j xh_j / C,
//   dinp = bf16(dresidual + rstd * (gy - xh * m)),  max |dinp|,
//   dweight[j] += sum_n dy[n, j] * xh[n, j]   (fp32)
// A workgroup of 256 threads takes one row at a time, each thread CPT
// 16-byte chunks of it (columns 8 * (t + 256 i)); the row's dot product is
// summed per wave, then over the four waves through LDS in a fixed order.
// Each workgroup walks a fixed set of rows and keeps its share of the weight
// gradient in registers (8 * CPT floats per thread); at the end it writes
// them as one row of `scratch` [workgroups, C].  A second kernel adds the
// rows of scratch in a fixed order to dweight, so the result does not depend
// on scheduling.  dinp may overwrite dresidual (each thread reads its chunks
// before it writes them).
constexpr int kBwdMaxGroups = 512;

static int rmsnorm_bwd_groups(int64_t N) { return (int)(N < kBwdMaxGroups ? N : kBwdMaxGroups); }

int64_t rmsnorm_bwd_scratch_floats(int64_t N, int C) { return N > 0 ? (int64_t)rmsnorm_bwd_groups(N) * C : 0; }

template <int CPT>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(uint16_t* dinp, float* __restrict__ scratch,
                                                          float* __restrict__ absmax, const uint16_t* dres,
                                                          const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ r,
                                                          const uint16_t* __restrict__ w,
                                                          const float* __restrict__ rstd, int64_t N, int C) {
    __shared__ float red[2][4];
    __shared__ float amax_red[4];
    const int t = threadIdx.x;
    const int lane = t & 63, wid = t >> 6;
    const int nch = C >> 3;
    float acc[CPT][8];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
    float amax = 0.0f;
    // the weight chunks are the same for every row
    const uint4* w4 = reinterpret_cast<const uint4*>(w);
    uint4 vw[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) vw[i] = w4[min(t + i * 256, nch - 1)];
    int parity = 0;
    for (int64_t row = blockIdx.x; row < N; row += gridDim.x, parity ^= 1) {
        const uint4* dy4 = reinterpret_cast<const uint4*>(dy + row * C);
        const uint4* r4 = reinterpret_cast<const uint4*>(r + row * C);
        const uint4* dr4 = reinterpret_cast<const uint4*>(dres + row * C);
        // every load of the row first; chunks past the row end load the last
        // chunk again and are left out
        uint4 vy[CPT], vr[CPT], vd[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = min(t + i * 256, nch - 1);
            vy[i] = dy4[c];
            vr[i] = r4[c];
            vd[i] = dr4[c];
        }
        const float rs = rstd[row];
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const uint32_t* yp = reinterpret_cast<const uint32_t*>(&vy[i]);
            const uint32_t* rp = reinterpret_cast<const uint32_t*>(&vr[i]);
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(&vw[i]);
            float p = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                p += (bf16lo(yp[q]) * bf16lo(wp[q])) * (bf16lo(rp[q]) * rs);
                p += (bf16hi(yp[q]) * bf16hi(wp[q])) * (bf16hi(rp[q]) * rs);
            }
            part += t + i * 256 < nch ? p : 0.0f;
        }
        part = wave_sum(part);
        // alternate two LDS slots by row so that one barrier per row suffices
        if (lane == 0) red[parity][wid] = part;
        __syncthreads();
        const float m = (((red[parity][0] + red[parity][1]) + red[parity][2]) + red[parity][3]) / (float)C;
        uint4* o4 = reinterpret_cast<uint4*>(dinp + row * C);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = t + i * 256;
            const bool ok = c < nch;
            const uint32_t* yp = reinterpret_cast<const uint32_t*>(&vy[i]);
            const uint32_t* rp = reinterpret_cast<const uint32_t*>(&vr[i]);
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(&vw[i]);
            const uint32_t* dp = reinterpret_cast<const uint32_t*>(&vd[i]);
            uint4 ov;
            uint32_t* op = reinterpret_cast<uint32_t*>(&ov);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float res[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float yv = h ? bf16hi(yp[q]) : bf16lo(yp[q]);
                    const float xh = (h ? bf16hi(rp[q]) : bf16lo(rp[q])) * rs;
                    const float gy = yv * (h ? bf16hi(wp[q]) : bf16lo(wp[q]));
                    res[h] = (h ? bf16hi(dp[q]) : bf16lo(dp[q])) + rs * (gy - xh * m);
                    acc[i][2 * q + h] += ok ? yv * xh : 0.0f;
                }
                op[q] = pack_bf16x2(res[0], res[1]);
                amax = ok ? absmax_acc(absmax_acc(amax, bf16lo(op[q])), bf16hi(op[q])) : amax;
            }
            if (ok) o4[c] = ov;
        }
    }
    float* srow = scratch + (int64_t)blockIdx.x * C;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = t + i * 256;
        if (c < nch) {
            reinterpret_cast<float4*>(srow + 8 * c)[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
            reinterpret_cast<float4*>(srow + 8 * c)[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
        }
    }
    if (absmax) block_absmax_commit(amax, amax_red, absmax);
}

// dweight[c] += sum over the scratch rows, in a fixed order: sixteen row
// partitions per column (partition p: rows p, p + 16, ..., eight loads in
// flight), each summed in row order, then combined in partition order.  A
// workgroup covers 16 columns.
constexpr int kReduceParts = 16;

// clear (nullable): an abs-max word set to zero by the first thread (the
// zero-once convention: the word whose consumer ran before this pass).
__global__ __launch_bounds__(256) void rmsnorm_dw_reduce_kernel(float* __restrict__ dweight,
                                                                const float* __restrict__ scratch, int rows, int C,
                                                                float* __restrict__ clear) {
    __shared__ float part[kReduceParts][16];
    const int col = threadIdx.x & 15, p = threadIdx.x >> 4;
    if (clear && blockIdx.x == 0 && threadIdx.x == 0) *clear = 0.0f;
    const int c = blockIdx.x * 16 + col;
    float s = 0.0f;
    if (c < C) {
        int w = p;
        for (; w + 7 * kReduceParts < rows; w += 8 * kReduceParts) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = scratch[(int64_t)(w + u * kReduceParts) * C + c];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; w < rows; w += kReduceParts) s += scratch[(int64_t)w * C + c];
    }
    part[p][col] = s;
    __syncthreads();
    if (p == 0 && c < C) {
        float t = part[0][col];
#pragma unroll
        for (int q = 1; q < kReduceParts; ++q) t += part[q][col];
        dweight[c] = dweight[c] + t;
    }
}

template <int CPT>
static void launch_rmsnorm_bwd_cpt(uint16_t* dinp, float* scratch, float* absmax, const uint16_t* dres,
                                   const uint16_t* dy, const uint16_t* r, const uint16_t* w, const float* rstd,
                                   int64_t N, int C, int groups, hipStream_t s) {
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<CPT>), dim3((unsigned)groups), dim3(256), 0, s, dinp, scratch, absmax,
                       dres, dy, r, w, rstd, N, C);
}

hipError_t launch_rmsnorm_bwd(uint16_t* dinp, float* dweight, float* scratch, const uint16_t* dres,
                              const uint16_t* dy, const uint16_t* r, const uint16_t* w, const float* rstd,
                              float* absmax, int64_t N, int C, hipStream_t s, bool clear_absmax, float* clear) {
    if (absmax && clear_absmax) {
        hipError_t e = launch_fill(absmax, 1, 0.0f, s);
        if (e != hipSuccess) return e;
    }
    if (N == 0) return clear ? launch_fill(clear, 1, 0.0f, s) : hipSuccess;
    const int groups = rmsnorm_bwd_groups(N);
    const int need = (C / 8 + 255) / 256;  // chunks per thread
    if (need <= 1) launch_rmsnorm_bwd_cpt<1>(dinp, scratch, absmax, dres, dy, r, w, rstd, N, C, groups, s);
    else if (need <= 2) launch_rmsnorm_bwd_cpt<2>(dinp, scratch, absmax, dres, dy, r, w, rstd, N, C, groups, s);
    else launch_rmsnorm_bwd_cpt<4>(dinp, scratch, absmax, dres, dy, r, w, rstd, N, C, groups, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rmsnorm_dw_reduce_kernel, dim3((unsigned)((C + 15) / 16)), dim3(256), 0, s, dweight, scratch,
                       groups, C, clear);
    return hipGetLastError();
}

}  // namespace ffn
