// MFMA GEMMs of the FFN block (gfx950): the fused gate+up projection with an
// optional SwiGLU + abs-max epilogue, and the down projection; bf16 operands or
// e4m3 operands with per-tensor fp32 scales (llmq llama_model.cpp, forward_qmm:
// matmul TN, scaled by weight.scale() and inp.Quant.scale(); _forward_block:
// up projection [2H, C], swiglu_forward, down projection [C, H]).
//
//   out[n, o] = sum_k x[n, k] * w[o, k]        (both operands K-contiguous)
//
// Tiling.  A workgroup of 4 waves owns a 256 (weight rows) x 256 (token rows)
// output tile and walks K in steps of 128 bytes per row (64 bf16 or 128 e4m3),
// so both dtypes share one LDS layout: per stage 256 rows x 128 B for each
// operand (64 KiB), two stages (128 KiB of the 160 KiB LDS).  Each wave owns a
// 128 x 128 sub-tile = 4 x 4 blocks of the 32x32 MFMA (v_mfma_f32_32x32x16_bf16
// or v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales), 256 fp32 accumulators
// per lane.  The weight is the MFMA's A operand, so each lane ends up holding
// four consecutive output features of one token: 8-byte bf16 stores.
//
// LDS layout.  Row r of a stage occupies 128 bytes = 8 chunks of 16 bytes;
// chunk c is stored at position c ^ (r & 7).  A fragment read (32 lanes on 32
// consecutive rows, one chunk each) then touches 8 distinct 16-byte positions
// in every group of 8 lanes: no bank conflicts.  Global loads put 8 lanes on
// the 8 chunks of one row (one 128-byte line).
//
// Pipeline.  The next K-step is loaded straight from global memory into the
// other LDS stage (global_load_lds_dwordx4, no registers) while the MFMAs
// consume the current stage; one wait + barrier per K-step.
//
// Tile order.  Workgroups are dealt to the 8 XCDs round-robin; the linear id is
// remapped so that each XCD receives a contiguous range of tiles, and inside it
// tiles are grouped 4 weight-panels wide, so the tiles resident on one XCD at a
// time share weight and token panels in that XCD's L2.
//
// SwiGLU fusion.  With fuse_swiglu the 256 weight rows of a tile are 128 gate
// rows and the 128 matching up rows, arranged so that every wave holds gate and
// up accumulators for the same (token, feature) pairs in the same registers:
// the epilogue rounds g and u to bf16, forms bf16(silu(g) * u), and folds the
// tile's abs-max into one atomic.
#include "common.h"
#include "launch.h"

namespace ffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kBM = 256;        // weight rows per tile
constexpr int kBN = 256;        // token rows per tile
constexpr int kRowBytes = 128;  // bytes per row per K-step
constexpr int kStage = (kBM + kBN) * kRowBytes;
constexpr int kGroupM = 4;

struct GemmArgs {
    void* out;
    float* absmax;
    const uint8_t* x;
    const uint8_t* w;
    const float* x_scale;
    const float* w_scale;
    int64_t N;     // token rows
    int K_bytes;   // bytes per operand row
    int O;         // weight rows (plain: output features; fused: 2H)
    int H;         // fused: intermediate size
    int ld_out;    // output row stride in elements
    int tiles_m;   // weight-row tiles
    int tiles_n;   // token-row tiles
};

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    int t = (T % 8 == 0) ? (b % 8) * (T / 8) + (b / 8) : b;
    const int per_group = kGroupM * tiles_n;
    const int group = t / per_group;
    const int first = group * kGroupM;
    const int gsize = min(tiles_m - first, kGroupM);
    const int r = t - group * per_group;
    tm = first + r % gsize;
    tn = r / gsize;
}

template <bool kFP8, bool kFused>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global -> LDS: direct loads (global_load_lds_dwordx4).  One wave
    // instruction fills 1 KiB of LDS = 8 rows; lane l lands at position
    // (row l/8, slot l%8) and so fetches chunk (l%8) ^ (l/8) of its row, which
    // realises the XOR swizzle.  Wave w fills rows [64 w, 64 w + 64) of both
    // operands.
    const int lrow = lane >> 3;
    const int lch = (lane & 7) ^ lrow;
    uint32_t a_off[8], b_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int R = wave * 64 + i * 8 + lrow;
        int wrow;
        if (kFused) {
            wrow = ((R & 64) ? a.H : 0) + tm * 128 + (R >> 7) * 64 + (R & 63);
        } else {
            wrow = min(tm * kBM + R, a.O - 1);
        }
        const int64_t xrow = min((int64_t)tn * kBN + R, a.N - 1);
        a_off[i] = (uint32_t)wrow * (uint32_t)a.K_bytes + (uint32_t)(lch << 4);
        b_off[i] = (uint32_t)xrow * (uint32_t)a.K_bytes + (uint32_t)(lch << 4);
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#define FFN_GLOAD(KT, ST)                                                                              \
    do {                                                                                               \
        const uint32_t kb_ = (uint32_t)(KT) * kRowBytes;                                               \
        uint8_t* sbase_ = lds + (ST) * kStage + wave * 64 * kRowBytes;                                 \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                             \
            __builtin_amdgcn_global_load_lds((const void*)(a.w + a_off[i_] + kb_),                     \
                (__attribute__((address_space(3))) void*)(sbase_ + i_ * 8 * kRowBytes), 16, 0, 0);     \
            __builtin_amdgcn_global_load_lds((const void*)(a.x + b_off[i_] + kb_),                     \
                (__attribute__((address_space(3))) void*)(sbase_ + kBM * kRowBytes + i_ * 8 * kRowBytes), \
                16, 0, 0);                                                                             \
        }                                                                                              \
    } while (0)

    // fragment rows of this lane
    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = fr & 7;

    const int KT = a.K_bytes / kRowBytes;
    FFN_GLOAD(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < KT) FFN_GLOAD(kt + 1, st ^ 1);
        const uint8_t* As = lds + st * kStage + (wm * 128 + fr) * kRowBytes;
        const uint8_t* Bs = lds + st * kStage + kBM * kRowBytes + (wn * 128 + fr) * kRowBytes;
        if (!kFP8) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int c = ((2 * kk + fh) ^ fsw) << 4;
                bf16x8_t fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fa[i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * kRowBytes + c);
                    fb[i] = *reinterpret_cast<const bf16x8_t*>(Bs + i * 32 * kRowBytes + c);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c0 = ((4 * kk + 2 * fh) ^ fsw) << 4;
                const int c1 = ((4 * kk + 2 * fh + 1) ^ fsw) << 4;
                i32x8_t fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 a0 = *reinterpret_cast<const uint4*>(As + i * 32 * kRowBytes + c0);
                    const uint4 a1 = *reinterpret_cast<const uint4*>(As + i * 32 * kRowBytes + c1);
                    const uint4 b0 = *reinterpret_cast<const uint4*>(Bs + i * 32 * kRowBytes + c0);
                    const uint4 b1 = *reinterpret_cast<const uint4*>(Bs + i * 32 * kRowBytes + c1);
                    fa[i] = i32x8_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    fb[i] = i32x8_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0,
                                                                                     127, 0, 127);
            }
        }
        // own direct loads for the next stage have landed, then everyone's
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
#undef FFN_GLOAD

    // ---- epilogue
    float s = 1.0f;
    if (kFP8) s = (*a.x_scale) * (*a.w_scale);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int64_t n_base = (int64_t)tn * kBN + wn * 128 + fr;
    if (!kFused) {
        const int o_base = tm * kBM + wm * 128 + fh * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n_base + j * 32;
            if (n >= a.N) continue;
            uint16_t* orow = out + n * a.ld_out;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int o = o_base + i * 32 + g * 8;
                    if (o < a.O) {
                        uint2 v;
                        v.x = pack_bf16x2(acc[i][j][4 * g + 0] * s, acc[i][j][4 * g + 1] * s);
                        v.y = pack_bf16x2(acc[i][j][4 * g + 2] * s, acc[i][j][4 * g + 3] * s);
                        *reinterpret_cast<uint2*>(orow + o) = v;
                    }
                }
        }
    } else {
        __shared__ float red[4];
        float amax = 0.0f;
        const int j_base = tm * 128 + wm * 64 + fh * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n_base + j * 32;
            const bool ok = n < a.N;
            uint16_t* orow = out + n * a.ld_out;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float hv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float gg = round_bf16(acc[i][j][4 * g + e] * s);
                        const float uu = round_bf16(acc[i + 2][j][4 * g + e] * s);
                        hv[e] = silu_mul(gg, uu);
                    }
                    uint2 v;
                    v.x = pack_bf16x2(hv[0], hv[1]);
                    v.y = pack_bf16x2(hv[2], hv[3]);
                    if (ok) {
                        amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(bf16lo(v.x)), __builtin_fabsf(bf16hi(v.x))),
                                                                     __builtin_fmaxf(__builtin_fabsf(bf16lo(v.y)), __builtin_fabsf(bf16hi(v.y)))));
                        *reinterpret_cast<uint2*>(orow + j_base + i * 32 + g * 8) = v;
                    }
                }
        }
        if (a.absmax) block_absmax_commit(amax, red, a.absmax);
    }
}

// Abs-max of a plain (unfused) GEMM output, when asked for: a separate pass.
hipError_t launch_gemm(void* out, float* absmax, const void* x, const float* x_scale, const void* w,
                       const float* w_scale, bool fp8, bool fuse_swiglu, int64_t N, int K, int O,
                       hipStream_t s) {
    if (absmax && (fuse_swiglu || N == 0)) {
        hipError_t e = launch_fill(absmax, 1, 0.0f, s);
        if (e != hipSuccess) return e;
    }
    if (N == 0) return hipSuccess;
    GemmArgs a;
    a.out = out;
    a.absmax = fuse_swiglu ? absmax : nullptr;
    a.x = static_cast<const uint8_t*>(x);
    a.w = static_cast<const uint8_t*>(w);
    a.x_scale = x_scale;
    a.w_scale = w_scale;
    a.N = N;
    a.K_bytes = K * (fp8 ? 1 : 2);
    a.O = O;
    a.H = O / 2;
    a.ld_out = fuse_swiglu ? O / 2 : O;
    a.tiles_m = fuse_swiglu ? (O / 2) / 128 : (O + kBM - 1) / kBM;
    a.tiles_n = (int)((N + kBN - 1) / kBN);
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(256);
    if (fp8) {
        if (fuse_swiglu) hipLaunchKernelGGL((gemm_kernel<true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<true, false>), grid, block, 0, s, a);
    } else {
        if (fuse_swiglu) hipLaunchKernelGGL((gemm_kernel<false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<false, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse_swiglu || !absmax) return e;
    return launch_absmax(absmax, static_cast<const uint16_t*>(out), N * (int64_t)O, s);
}

}  // namespace ffn
