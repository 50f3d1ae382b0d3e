// MFMA GEMMs of the FFN block (gfx950): the fused gate+up projection with an
// optional SwiGLU + abs-max epilogue, and the down projection; bf16 operands or
// e4m3 operands with per-tensor fp32 scales (llmq llama_model.cpp, forward_qmm:
// matmul TN, scaled by weight.scale() and inp.Quant.scale(); _forward_block:
// up projection [2H, C], swiglu_forward, down projection [C, H]).
//
//   out[n, o] = sum_k x[n, k] * w[o, k]        (both operands K-contiguous)
//
// Tiling.  A workgroup of 8 waves (two per SIMD) owns a 256 (weight rows) x
// 256 (token rows) output tile and walks K in steps of 64 bytes per row (32
// bf16 or 64 e4m3), so both dtypes share one LDS layout: per stage 256 rows x
// 64 B for each operand (32 KiB).  The waves form a 2 x 4 grid; each owns a
// 128 x 64 sub-tile = 4 x 2 blocks of the 32x32 MFMA (v_mfma_f32_32x32x16_bf16
// or v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales), 128 fp32 accumulators
// per lane.  The weight is the MFMA's A operand, so each lane ends up holding
// four consecutive output features of one token: 8-byte bf16 stores.
//
// LDS layout.  Row r of a stage occupies 64 bytes = 4 chunks of 16 bytes;
// chunk c is stored at position c ^ ((r / 4) % 4).  The LDS serves a 16-byte
// read 16 lanes at a time across 64 banks (256 bytes); a fragment read puts 16
// lanes on 16 consecutive rows at one chunk, and the rows that share a bank
// offset (r, r+4, r+8, r+12) land on 4 different positions: no bank
// conflicts.  Global loads put 4 lanes on the 4 chunks of one row.
//
// Pipeline.  K-steps are loaded straight from global memory into a ring of
// five LDS stages (global_load_lds_dwordx4, no registers), three to four
// steps ahead of the MFMAs, the load instructions interleaved with the MFMAs.
// Steps are consumed in pairs: one counted wait (vmcnt) for this wave's loads
// of the pair, one barrier per two K-steps.
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
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;        // weight rows per tile
constexpr int kBN = 256;        // token rows per tile
constexpr int kRowBytes = 64;   // bytes per row per K-step (32 bf16 or 64 e4m3)
constexpr int kStages = 5;      // LDS ring of K-steps: 5 x 32 KiB = all 160 KiB
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

// One wave-wide direct load: each lane's 16 bytes at gptr land in LDS at
// lds_base + 16 * lane.  Issued as inline assembly so that the compiler does
// not treat every later LDS read as dependent on it (it would otherwise wait
// for all outstanding loads before each read); the kernel orders these loads
// against its LDS reads itself, with counted vmcnt waits and barriers.
__device__ __forceinline__ void load_lds16(const void* gptr, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gptr), "s"(lds_base)
        : "memory");
}

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

template <int kWaves>
struct WaveShape {
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kNB = kWaves == 4 ? 4 : 2;    // 32-column blocks per wave along the tokens
    static constexpr int kWN = kWaves / 2;             // waves along the tokens
    static constexpr int kLI = 256 / kWaves / 16;      // load instructions per operand per K-step
};

template <bool kFP8, bool kFused, int kWaves>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves),
                          amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void gemm_kernel(GemmArgs a) {
    using WS = WaveShape<kWaves>;
    constexpr int kNB = WS::kNB, kLI = WS::kLI;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
    static_assert(kStages * kStage <= 160 * 1024, "LDS ring exceeds the 160 KiB of a CU");

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave / WS::kWN, wn = wave % WS::kWN;

    // ---- global -> LDS: direct loads (global_load_lds_dwordx4).  One wave
    // instruction fills 1 KiB of LDS = 16 rows of 64 bytes; lane l lands at
    // (row l/4, slot l%4) and so fetches chunk (l%4) ^ ((row/4)%4) of its row,
    // which realises the XOR swizzle.  Wave w fills rows [16 kLI w, 16 kLI (w+1))
    // of both operands: kLI instructions each.
    const int lrow = lane >> 2;
    const int lch = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t a_off[kLI], b_off[kLI];
#pragma unroll
    for (int i = 0; i < kLI; ++i) {
        const int R = wave * 16 * kLI + i * 16 + lrow;
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

    f32x16_t acc[4][kNB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // LDS byte address of this wave's first row (wave-uniform: an SGPR)
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + wave * 16 * kLI * kRowBytes);
#define FFN_GLOAD(KT, ST)                                                                              \
    do {                                                                                               \
        const uint32_t kb_ = (uint32_t)(KT) * kRowBytes;                                               \
        const uint32_t sb_ = lds_wave + (uint32_t)((ST) * kStage);                                     \
        _Pragma("unroll") for (int i_ = 0; i_ < kLI; ++i_) {                                           \
            load_lds16(a.w + a_off[i_] + kb_, sb_ + i_ * 16 * kRowBytes);                              \
            load_lds16(a.x + b_off[i_] + kb_, sb_ + kBM * kRowBytes + i_ * 16 * kRowBytes);            \
        }                                                                                              \
    } while (0)

    // fragment rows of this lane: row fr of each 32-row block, K half fh
    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = (fr >> 2) & 3;
    // Fragments of one K-step.  bf16: per 32-row block two 16-byte pieces,
    // one per 16-value K sub-step (chunk 2*p + fh).  e4m3: per block the lane's
    // 32 bytes (chunks 2*fh and 2*fh + 1) for one 32x32x64 MFMA.
    int coff[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) coff[p] = ((kFP8 ? (2 * fh + p) : (2 * p + fh)) ^ fsw) << 4;
    const int a_row = (wm * 128 + fr) * kRowBytes;
    const int b_row = kBM * kRowBytes + (wn * kNB * 32 + fr) * kRowBytes;

    const int KT = a.K_bytes / kRowBytes;

    // One of the 2*kLI load instructions of K-step `step` (A parts first).
    auto load_part = [&](int step, int part) {
        const uint32_t kb = (uint32_t)step * kRowBytes;
        const uint32_t sb = lds_wave + (uint32_t)((step % kStages) * kStage);
        if (part < kLI) load_lds16(a.w + a_off[part] + kb, sb + part * 16 * kRowBytes);
        else load_lds16(a.x + b_off[part - kLI] + kb, sb + kBM * kRowBytes + (part - kLI) * 16 * kRowBytes);
    };

    // The MFMAs of K-step kt.  After each 32-row block of A one load of
    // K-step `ld` is issued (parts ld_part0 ..), so the ring refills spread
    // over the MFMAs instead of arriving as one burst.
    auto compute_step = [&](int kt, int ld, int ld_part0) {
        const uint8_t* base = lds + (kt % kStages) * kStage;
        i32x4_t fa[4][2], fb[kNB][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i][p] = *reinterpret_cast<const i32x4_t*>(base + a_row + i * 32 * kRowBytes + coff[p]);
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                fb[j][p] = *reinterpret_cast<const i32x4_t*>(base + b_row + j * 32 * kRowBytes + coff[p]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!kFP8) {
#pragma unroll
                for (int p = 0; p < 2; ++p)
#pragma unroll
                    for (int j = 0; j < kNB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, fa[i][p]), __builtin_bit_cast(bf16x8_t, fb[j][p]),
                            acc[i][j], 0, 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        __builtin_shufflevector(fa[i][0], fa[i][1], 0, 1, 2, 3, 4, 5, 6, 7),
                        __builtin_shufflevector(fb[j][0], fb[j][1], 0, 1, 2, 3, 4, 5, 6, 7), acc[i][j], 0, 0,
                        0, 127, 0, 127);
            }
            if (ld < KT && ld_part0 + i < 2 * kLI) load_part(ld, ld_part0 + i);
        }
        // parts beyond four per step (kLI > 2)
#pragma unroll
        for (int q = ld_part0 + 4; q < 2 * kLI; ++q)
            if (ld < KT) load_part(ld, q);
    };

    // K-steps go through the ring in pairs.  Before pair (k, k+1) this wave
    // has issued the loads of steps up to k+2; its loads of k and k+1 have
    // landed once at most those of k+2 are outstanding.  The barrier that
    // follows extends that to every wave and retires every read of steps k-2
    // and k-1, whose stages then take steps k+3 (issued during step k) and k+4
    // (during step k+1).
#pragma unroll
    for (int s = 0; s < 3; ++s)
        if (s < KT) FFN_GLOAD(s, s);
    for (int kp = 0; kp < KT; kp += 2) {
        if (min(kp + 2, KT - 1) > min(kp + 1, KT - 1)) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLI) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        compute_step(kp, kp + 3, 0);
        if (kp + 1 < KT) compute_step(kp + 1, kp + 4, 0);
    }
#undef FFN_GLOAD

    // ---- epilogue
    float s = 1.0f;
    if (kFP8) s = (*a.x_scale) * (*a.w_scale);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int64_t n_base = (int64_t)tn * kBN + wn * kNB * 32 + fr;
    if (!kFused) {
        const int o_base = tm * kBM + wm * 128 + fh * 4;
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
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
        // the ring is free once every wave is past its last MFMA reads
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds);
        float amax = 0.0f;
        const int j_base = tm * 128 + wm * 64 + fh * 4;
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
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

constexpr int kGemmWaves = 8;

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
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(WaveShape<kGemmWaves>::kThreads);
    if (fp8) {
        if (fuse_swiglu) hipLaunchKernelGGL((gemm_kernel<true, true, kGemmWaves>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<true, false, kGemmWaves>), grid, block, 0, s, a);
    } else {
        if (fuse_swiglu) hipLaunchKernelGGL((gemm_kernel<false, true, kGemmWaves>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<false, false, kGemmWaves>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse_swiglu || !absmax) return e;
    return launch_absmax(absmax, static_cast<const uint16_t*>(out), N * (int64_t)O, s);
}

}  // namespace ffn
