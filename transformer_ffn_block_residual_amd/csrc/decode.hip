// FP8-weight, bf16-activation decode GEMVs (metrale dense_ffn_decode.rs,
// DenseFfnLayer::forward, FP8 arm): the dual gate/up GEMV with per-row scales,
// whose epilogue applies silu(g) * u (the split-SiLU arm's silu_mul, fused so
// the intermediate g and u never leave registers), then the down GEMV.
//
//   g[m,n] = bf16(sg[n] * sum_k Wg[n,k] x[m,k]),  u likewise
//   h[m,n] = bf16(silu(g) * u)
//   y[m,c] = bf16(sd[c] * sum_n Wd[c,n] h[m,n])
//
// The weights are streamed once from HBM: every wave owns RPW weight rows (of
// each matrix in the dual pass) and walks K in 1 KiB segments, one 16-byte
// load (16 e4m3 codes) per lane per row per segment, two segments in flight.
// Codes are decoded with v_cvt_pk_f32_fp8 (exact) and accumulated in fp32
// against the activations, which are re-read per segment from L1/L2 (they are
// a few KiB and shared by every wave).  A row's partial sums are reduced across
// the wave at the end; lane m writes token m.
#include "common.h"
#include "launch.h"

namespace ffn {

constexpr int kSeg = 1024;  // bytes of one weight row per wave-wide 16-byte load

template <int MT>
__device__ __forceinline__ void load_act(float (&xv)[MT][16], const uint16_t* __restrict__ x, int64_t ldx, int k,
                                         bool ok, int M) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
        if (ok && m < M) {
            const uint4* p = reinterpret_cast<const uint4*>(x + m * ldx + k);
            v0 = p[0];
            v1 = p[1];
        }
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            xv[m][2 * q] = bf16lo(w[q]);
            xv[m][2 * q + 1] = bf16hi(w[q]);
        }
    }
}

template <int MT>
__device__ __forceinline__ void fma_row(float (&acc)[MT], const uint4 wq, const float (&xv)[MT][16]) {
    const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const f32x2_t lo = e4m3x2_to_f32(w[q], false);
        const f32x2_t hi = e4m3x2_to_f32(w[q], true);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc[m] = __builtin_fmaf(lo[0], xv[m][4 * q + 0], acc[m]);
            acc[m] = __builtin_fmaf(lo[1], xv[m][4 * q + 1], acc[m]);
            acc[m] = __builtin_fmaf(hi[0], xv[m][4 * q + 2], acc[m]);
            acc[m] = __builtin_fmaf(hi[1], xv[m][4 * q + 3], acc[m]);
        }
    }
}

// kDual: rows of w0 (gate) and w1 (up) with the SiLU epilogue -> out = h [M, rows].
// else : rows of w0 (down) -> out = y [M, rows].
template <int MT, int RPW, bool kDual>
__global__ __launch_bounds__(256) void gemv_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ x,
                                                   const uint8_t* __restrict__ w0, const float* __restrict__ s0,
                                                   const uint8_t* __restrict__ w1, const float* __restrict__ s1,
                                                   int M, int K, int rows) {
    constexpr int NMAT = kDual ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int row0 = wave_g * RPW;
    if (row0 >= rows) return;

    float acc[NMAT][RPW][MT];
#pragma unroll
    for (int a = 0; a < NMAT; ++a)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[a][r][m] = 0.0f;

    const uint8_t* wp[NMAT][RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int row = min(row0 + r, rows - 1);
        wp[0][r] = w0 + (int64_t)row * K;
        if (kDual) wp[NMAT - 1][r] = w1 + (int64_t)row * K;
    }

    const int nseg = (K + kSeg - 1) / kSeg;
    for (int sg = 0; sg < nseg; ++sg) {
        const int k = sg * kSeg + lane * 16;
        const bool ok = k < K;
        uint4 wq[NMAT][RPW];
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                wq[a][r] = ok ? *reinterpret_cast<const uint4*>(wp[a][r] + k) : make_uint4(0, 0, 0, 0);
        float xv[MT][16];
        load_act<MT>(xv, x, K, k, ok, M);
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int r = 0; r < RPW; ++r) fma_row<MT>(acc[a][r], wq[a][r], xv);
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int row = row0 + r;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float v0 = wave_sum(acc[0][r][m]);
            float v1 = kDual ? wave_sum(acc[NMAT - 1][r][m]) : 0.0f;
            if (lane == m && row < rows && m < M) {
                float o;
                if (kDual) {
                    const float g = round_bf16(s0[row] * v0);
                    const float u = round_bf16(s1[row] * v1);
                    o = silu_mul(g, u);
                } else {
                    o = s0[row] * v0;
                }
                out[(int64_t)m * rows + row] = (uint16_t)(pack_bf16x2(o, 0.0f) & 0xffffu);
            }
        }
    }
}

template <int MT>
static hipError_t launch_decode_mt(uint16_t* out, uint16_t* h, const uint16_t* x, const uint8_t* wg,
                                   const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd,
                                   const float* sd, int M, int C, int H, hipStream_t s) {
    constexpr int RPW_DUAL = MT <= 2 ? 4 : (MT <= 8 ? 2 : 1);
    constexpr int RPW_DOWN = MT <= 2 ? 2 : 1;
    const int waves_dual = (H + RPW_DUAL - 1) / RPW_DUAL;
    hipLaunchKernelGGL((gemv_kernel<MT, RPW_DUAL, true>), dim3((waves_dual + 3) / 4), dim3(256), 0, s, h, x, wg,
                       sg, wu, su, M, C, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int waves_down = (C + RPW_DOWN - 1) / RPW_DOWN;
    hipLaunchKernelGGL((gemv_kernel<MT, RPW_DOWN, false>), dim3((waves_down + 3) / 4), dim3(256), 0, s, out, h,
                       wd, sd, nullptr, nullptr, M, H, C);
    return hipGetLastError();
}

hipError_t launch_decode(uint16_t* out, uint16_t* h, const uint16_t* x, const uint8_t* wg, const float* sg,
                         const uint8_t* wu, const float* su, const uint8_t* wd, const float* sd, int M, int C,
                         int H, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (M == 1) return launch_decode_mt<1>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
    if (M <= 2) return launch_decode_mt<2>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
    if (M <= 4) return launch_decode_mt<4>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
    if (M <= 8) return launch_decode_mt<8>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
    if (M <= 16) return launch_decode_mt<16>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
    return launch_decode_mt<32>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
}

}  // namespace ffn
