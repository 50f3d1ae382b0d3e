// MFMA GEMMs of the FFN block (gfx950): the fused gate+up projection with an
// optional SwiGLU + abs-max epilogue, and the down projection; bf16 operands or
// e4m3 operands with per-tensor fp32 scales (llmq llama_model.cpp, forward_qmm:
// matmul TN, scaled by weight.scale() and inp.Quant.scale(); _forward_block:
// up projection [2H, C], swiglu_forward, down projection [C, H]).
//
//   out[n, o] = sum_k x[n, k] * w[o, k]        (both operands K-contiguous)
//
// Tiling.  A workgroup of 4 waves (one per SIMD) owns a 256 (weight rows) x
// 256 (token rows) output tile and walks K in steps of 64 bytes per row (32
// bf16 or 64 e4m3), so both dtypes share one LDS layout: per stage 256 rows x
// 64 B for each operand (32 KiB).  The waves form a 2 x 2 grid; each owns a
// 128 x 128 sub-tile = 4 x 4 blocks of the 32x32 MFMA (v_mfma_f32_32x32x16_bf16
// or v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales): 256 fp32 accumulators
// per lane, which live in the accumulation registers.  The weight is the MFMA's
// A operand, so each lane ends up holding four consecutive output features of
// one token: 8-byte bf16 stores.
//
// LDS layout.  Row r of a stage occupies 64 bytes = 4 chunks of 16 bytes;
// chunk c is stored at position c ^ ((r / 4) % 4).  The LDS serves a 16-byte
// read 16 lanes at a time across 64 banks (256 bytes); a fragment read puts 16
// lanes on 16 consecutive rows at one chunk, and the rows that share a bank
// offset (r, r+4, r+8, r+12) land on 4 different positions: no bank
// conflicts.  Global loads put 4 lanes on the 4 chunks of one row.
//
// Pipeline.  K-steps are loaded straight from global memory into a ring of
// five LDS stages (global_load_lds_dwordx4, no registers), four steps ahead of
// the MFMAs.  The fragments of step k+1 are read from LDS into a second
// register set while the MFMAs of step k run, so a step's MFMAs never wait for
// the LDS; one counted wait (vmcnt) and one barrier per step publish the next
// stage and retire the oldest.  Inside a step the MFMAs, fragment reads and
// global loads are issued in a fixed interleave (the compiler's scheduler is
// fenced off), one MFMA at a time.
//
// Tile order.  Workgroups are dealt to the 8 XCDs round-robin; the linear id is
// remapped so that each XCD receives a contiguous range of tiles, and inside it
// tiles are grouped 4 weight-panels wide, so the tiles resident on one XCD at a
// time share weight and token panels in that XCD's L2.
//
// SwiGLU fusion.  With fuse_swiglu the 256 weight rows of a tile are 128 gate
// rows and the 128 matching up rows, arranged so that every wave holds gate and
// up accumulators for the same (token, feature) pairs in matching registers:
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
constexpr int kAhead = 4;       // K-steps in flight ahead of the one being multiplied
constexpr int kThreads = 256;   // 4 waves
constexpr int kLoads = kBM / 4 / 16;  // load instructions per operand per wave per K-step
constexpr int kBlockBytes = 32 * kRowBytes;  // one 32-row MFMA block of a stage
constexpr int kGroupM = 4;
static_assert(kAhead < kStages, "a stage is refilled only after the barrier that retires it");

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

// One wave-wide direct load: lane l's 16 bytes at base + off land in LDS at
// lds_addr + 16 l.  Issued as inline assembly so that the compiler does not
// treat every later LDS read as dependent on it (it would otherwise wait for
// all outstanding loads before each read); the kernel orders these loads
// against its LDS reads itself, with counted vmcnt waits and barriers.
__device__ __forceinline__ void load_lds16(uint32_t off, const uint8_t* base, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(off), "s"(base), "s"(lds_addr)
        : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// Register fragments of one K-step: per 32-row block of A (weights) and B
// (tokens) two 16-byte pieces.  bf16: piece p feeds the p-th 16-value K
// sub-step (chunk 2p + fh).  e4m3: the two pieces are the lane's 32 bytes
// (chunks 2fh, 2fh + 1) of one 32x32x64 MFMA.
struct Frags {
    i32x4_t a[4][2];
    i32x4_t b[4][2];
};

// Where a wave's loads and reads of a K-step go.
struct StepIO {
    const uint8_t* lds;     // the ring (generic pointer)
    uint32_t lds_wave;      // LDS address of this wave's first load row in stage 0
    uint32_t a_off[kLoads];  // byte offsets of this lane's load rows in w and x
    uint32_t b_off[kLoads];
    int a_rd[2], b_rd[2];   // byte offsets of this lane's fragment pieces in a stage
};

__device__ __forceinline__ void read_frags(Frags& f, const StepIO& io, int step) {
    const uint8_t* st = io.lds + (step % kStages) * kStage;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int blk = (r & 7) >> 1, p = r & 1;
        if (r < 8) f.a[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.a_rd[p] + blk * kBlockBytes);
        else f.b[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.b_rd[p] + blk * kBlockBytes);
    }
}

// Load instruction l (0 .. 2 kLoads - 1; A first) of K-step `step`.
__device__ __forceinline__ void load_part(const GemmArgs& a, const StepIO& io, int step, int l) {
    const uint32_t kb = (uint32_t)step * kRowBytes;
    const uint32_t st = io.lds_wave + (uint32_t)((step % kStages) * kStage);
    if (l < kLoads) load_lds16(io.a_off[l], a.w + kb, st + l * 16 * kRowBytes);
    else load_lds16(io.b_off[l - kLoads], a.x + kb, st + kBM * kRowBytes + (l - kLoads) * 16 * kRowBytes);
}

// The MFMAs of K-step k from `cur`; with kRead the fragments of step k + 1 are
// read into `nxt` meanwhile, with kLoad the loads of step k + kAhead issued.
template <bool kFP8, bool kLoad, bool kRead>
__device__ __forceinline__ void k_step(f32x16_t (&acc)[4][4], const Frags& cur, Frags& nxt, const GemmArgs& a,
                                       const StepIO& io, int k) {
    constexpr int kM = kFP8 ? 16 : 32;  // MFMAs per step
    constexpr int kPerRead = kM / 16, kPerLoad = kM / (2 * kLoads);
    const uint8_t* st = io.lds + ((k + 1) % kStages) * kStage;
    const int kl = k + kAhead;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
        if (kRead && m % kPerRead == 0) {
            const int r = m / kPerRead, blk = (r & 7) >> 1, p = r & 1;
            if (r < 8) nxt.a[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.a_rd[p] + blk * kBlockBytes);
            else nxt.b[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.b_rd[p] + blk * kBlockBytes);
        }
        if (kFP8) {
            const int i = m >> 2, j = m & 3;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                __builtin_shufflevector(cur.a[i][0], cur.a[i][1], 0, 1, 2, 3, 4, 5, 6, 7),
                __builtin_shufflevector(cur.b[j][0], cur.b[j][1], 0, 1, 2, 3, 4, 5, 6, 7), acc[i][j], 0, 0, 0,
                127, 0, 127);
        } else {
            const int i = m >> 3, j = (m >> 1) & 3, p = m & 1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cur.a[i][p]),
                                                                __builtin_bit_cast(bf16x8_t, cur.b[j][p]),
                                                                acc[i][j], 0, 0, 0);
        }
        if (kLoad && m % kPerLoad == kPerLoad - 1) load_part(a, io, kl, m / kPerLoad);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool kFP8, bool kFused>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
    static_assert(kStages * kStage <= 160 * 1024, "LDS ring exceeds the 160 KiB of a CU");

    int tm, tn;
    tile_coords(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    StepIO io;
    io.lds = lds;
    // ---- global -> LDS.  One wave instruction fills 1 KiB of a stage = 16
    // rows of 64 bytes; lane l lands at (row l/4, slot l%4) and so fetches
    // chunk (l%4) ^ ((row/4)%4) of its row, which realises the XOR swizzle.
    // Wave w fills rows [64 w, 64 w + 64) of both operands.
    const int lrow = lane >> 2;
    const int lch = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int R = wave * 16 * kLoads + i * 16 + lrow;
        int wrow;
        if (kFused) {
            wrow = ((R & 64) ? a.H : 0) + tm * 128 + (R >> 7) * 64 + (R & 63);
        } else {
            wrow = min(tm * kBM + R, a.O - 1);
        }
        const int64_t xrow = min((int64_t)tn * kBN + R, a.N - 1);
        io.a_off[i] = (uint32_t)wrow * (uint32_t)a.K_bytes + (uint32_t)(lch << 4);
        io.b_off[i] = (uint32_t)xrow * (uint32_t)a.K_bytes + (uint32_t)(lch << 4);
    }
    io.lds_wave = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds + wave * 16 * kLoads * kRowBytes);

    // fragment rows of this lane: row fr of each 32-row block, K half fh
    const int fr = lane & 31, fh = lane >> 5;
    const int fsw = (fr >> 2) & 3;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int coff = ((kFP8 ? (2 * fh + p) : (2 * p + fh)) ^ fsw) << 4;
        io.a_rd[p] = (wm * 128 + fr) * kRowBytes + coff;
        io.b_rd[p] = kBM * kRowBytes + (wn * 128 + fr) * kRowBytes + coff;
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // K-steps: KT is even (the ABI requires K % 128 == 0 elements).  Step k
    // lives in stage k % 5.  Before the MFMAs of step k, steps k and k + 1 are
    // in LDS and visible to every wave (the fragments of k are in registers),
    // and this wave has issued the loads of steps up to k + 3.  During step k
    // it issues the loads of step k + 4 into the stage of step k - 1, whose
    // fragments every wave finished reading before the barrier that closed
    // step k - 1; after step k it waits for its loads of step k + 2 and meets
    // the others at the barrier.
    const int KT = a.K_bytes / kRowBytes;
    Frags f0, f1;
    const int n0 = min(kAhead, KT);
#pragma unroll
    for (int s = 0; s < kAhead; ++s)
        if (s < n0)
#pragma unroll
            for (int l = 0; l < 2 * kLoads; ++l) load_part(a, io, s, l);
    if (n0 == kAhead) wait_vmcnt<2 * kLoads * (kAhead - 2)>();
    else wait_vmcnt<0>();
    barrier();
    read_frags(f0, io, 0);

    int k = 0;
    for (; k + kAhead < KT; k += 2) {
        k_step<kFP8, true, true>(acc, f0, f1, a, io, k);
        wait_vmcnt<2 * kLoads * (kAhead - 2)>();
        barrier();
        k_step<kFP8, true, true>(acc, f1, f0, a, io, k + 1);
        wait_vmcnt<2 * kLoads * (kAhead - 2)>();
        barrier();
    }
    // the last steps issue no loads: KT - 4 and KT - 3 (when KT >= 4) drain
    // the loads in flight, KT - 2 and KT - 1 need no more barriers
    static_assert(kAhead == 4, "the drain below is written for four steps in flight");
    if (k + 2 < KT) {
        k_step<kFP8, false, true>(acc, f0, f1, a, io, k);
        wait_vmcnt<2 * kLoads>();
        barrier();
        k_step<kFP8, false, true>(acc, f1, f0, a, io, k + 1);
        wait_vmcnt<0>();
        barrier();
        k += 2;
    }
    k_step<kFP8, false, true>(acc, f0, f1, a, io, k);
    k_step<kFP8, false, false>(acc, f1, f0, a, io, k + 1);

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
        // the ring is free once every wave is past its last MFMA reads
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds);
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
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(kThreads);
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
