// FP8-weight, bf16-activation decode GEMVs (metrale dense_ffn_decode.rs,
// DenseFfnLayer::forward, FP8 arm): the dual gate/up GEMV with per-row scales,
// whose epilogue applies silu(g) * u (the split-SiLU arm's silu_mul, fused so
// the intermediate g and u never leave registers), then the down GEMV.
//
//   g[m,n] = bf16(sg[n] * sum_k Wg[n,k] x[m,k]),  u likewise
//   h[m,n] = bf16(silu(g) * u)
//   y[m,c] = bf16(sd[c] * sum_n Wd[c,n] h[m,n])
//
// Both passes stream their weights from HBM once and are bound by it.  For
// one to four tokens the lanes split K instead (gemv_small_kernel below).  For
// more, a workgroup of 8 waves owns 16 weight rows (of each matrix in the dual pass);
// its waves split K into 256-byte chunks, dealt round-robin.  Per chunk a lane
// loads four 16-byte pieces of one row, the 4 lanes of a row covering 64
// contiguous bytes per load instruction; the codes are widened to bf16 with
// v_cvt_scalef32_pk_bf16_fp8 (exact: every e4m3 value is a bf16 value) and fed
// as the A operand of v_mfma_f32_16x16x32_bf16, whose B operand holds the
// matching activations of up to 16 tokens (zero beyond M).  The MFMA's K order
// is free as long as A and B agree, so each lane's 8 codes per MFMA are simply
// the 8 it loaded.  The eight partial 16 x 16 results are summed through LDS;
// the row scale multiplies the finished fp32 sum.  The packed form of the same
// kernel reads weights re-laid in 1 KiB pieces (16 rows x 64 codes, piece-major
// over the 16-row blocks) and activations re-laid in operand order, one
// contiguous KiB per load instruction (see kPacked).
#include "common.h"
#include "launch.h"

namespace ffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// waves per workgroup per pass; row blocks per workgroup of the dual pass
// when several tokens share each weight (activation reuse)
constexpr int kDualWaves = 8, kDownWaves = 8, kDualRB = 1;
constexpr int kChunk = 256;  // K bytes (= e4m3 codes) per wave per step
constexpr int kPieces = kChunk / 64;  // 16-byte loads per lane per row per step

// 8 e4m3 codes (two dwords) -> 8 bf16 in MFMA operand order.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    const bf16x2_t a = e4m3x2_to_bf16(w0, false), b = e4m3x2_to_bf16(w0, true);
    const bf16x2_t c = e4m3x2_to_bf16(w1, false), d = e4m3x2_to_bf16(w1, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A raw buffer resource over `bytes` bytes at p, and a 16-byte load from it
// at voff (per lane) + soff (uniform); the streaming loops keep their bases
// and piece offsets in scalar registers this way.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// kDual: rows of w0 (gate) and w1 (up) with the SiLU epilogue -> out = h [M, rows].
// else : rows of w0 (down) -> out = y [M, rows].  x: [M, K] bf16.  TB = 16-token
// blocks (M <= 16 * TB); RB = 16-row blocks per workgroup (each activation
// fragment is multiplied into RB * NMAT row blocks).
// kPacked: the weights are in the packed decode layout (1 KiB pieces of 16
// rows x 64 codes, in which lane l's 16 bytes are row l % 16, codes
// 16 (l / 16) .. + 15 of those 64, piece kc of row block rb at KiB
// kc * rows / 16 + rb: one contiguous KiB per load instruction, landing in
// MFMA operand order), x is in fragment order (token
// block tb, fragment f, lane l: 8 values of token 16 tb + l % 16 at
// k = 64 (f / 2) + 16 (l / 16) + 8 (f % 2) + 0..7, zero past M: one contiguous
// KiB per B operand), and the dual pass also writes h in fragment order to hp
// (all 16 tokens of each block; zero past M) for the down pass.
template <bool kDual, int TB, int RB, int kWaves, bool kPacked = false>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(
    uint16_t* __restrict__ out, uint16_t* __restrict__ hp, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ w0, const float* __restrict__ s0, const uint8_t* __restrict__ w1,
    const float* __restrict__ s1, int M, int K, int rows) {
    constexpr int NMAT = kDual ? 2 : 1;
    __shared__ f32x4_t red[kWaves][RB][NMAT][TB][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * 16 * RB;
    const int lr = lane & 15;   // weight row within a block / token within a token block
    const int lq = lane >> 4;   // which 16-byte quarter of each 64-byte piece

    const uint8_t* wrow[RB][NMAT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (kPacked) {
            // rows % 16 == 0: piece 0 of the block; piece kc lies kc * rows / 16 KiB on
            const int64_t blk = (int64_t)((row0 + rb * 16) / 16) * 1024 + lane * 16;
            wrow[rb][0] = w0 + blk;
            if (kDual) wrow[rb][NMAT - 1] = w1 + blk;
        } else {
            const int row = min(row0 + rb * 16 + lr, rows - 1);
            wrow[rb][0] = w0 + (int64_t)row * K + lq * 16;
            if (kDual) wrow[rb][NMAT - 1] = w1 + (int64_t)row * K + lq * 16;
        }
    }
    const uint16_t* xrow[TB];
    bool tok_ok[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int tok = tb * 16 + lr;
        tok_ok[tb] = kPacked || tok < M;  // the fragment-order copy is zero past M
        xrow[tb] = kPacked ? x + (int64_t)tb * 16 * K + lane * 8 : x + (int64_t)min(tok, M - 1) * K + lq * 16;
    }

    f32x4_t acc[RB][NMAT][TB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[rb][m][tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Chunks go to the waves round-robin.  Each workgroup starts its walk
    // along K at a different chunk, so the rows that the workgroups stream at
    // one moment are not all at the same column offset (with power-of-two row
    // lengths those addresses crowd the same HBM channels).  Packed weights
    // are piece-major: there every workgroup starts at chunk 0, so that the
    // workgroups sweep each matrix in address order (about 1 us faster).
    const int nchunks = (K + kChunk - 1) / kChunk;  // K % 128 == 0: the last chunk may be half
    const int rot = kPacked ? 0 : (int)(((unsigned)blockIdx.x * 5u) % (unsigned)nchunks);
    for (int cw = wave; cw < nchunks; cw += kWaves) {
        const int c = cw + rot < nchunks ? cw + rot : cw + rot - nchunks;
        const int kb = c * kChunk;
        // piece i of a row: bytes [kb + 64 i + 16 lq, +16): the 4 lanes of a
        // row read 64 contiguous bytes per instruction
        uint4 wq[RB][NMAT][kPieces];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < kPieces; ++i)
                    wq[rb][m][i] = (kb + 64 * i < K)
                                       ? *reinterpret_cast<const uint4*>(
                                             wrow[rb][m] + (kPacked ? (int64_t)(kb + 64 * i) * rows : kb + 64 * i))
                                       : make_uint4(0, 0, 0, 0);
        // the matching activations: 8 values per MFMA, piece i half q
        bf16x8_t xb[TB][kPieces][2];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < kPieces; ++i)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (tok_ok[tb] && kb + 64 * i < K)
                        v = *reinterpret_cast<const uint4*>(
                            xrow[tb] + (kPacked ? (int64_t)((kb + 64 * i) / 32 + q) * 512 : kb + 64 * i + 8 * q));
                    xb[tb][i][q] = __builtin_bit_cast(bf16x8_t, v);
                }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < kPieces; ++i) {
                    const bf16x8_t a0 = e4m3x8_to_bf16(wq[rb][m][i].x, wq[rb][m][i].y);
                    const bf16x8_t a1 = e4m3x8_to_bf16(wq[rb][m][i].z, wq[rb][m][i].w);
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        acc[rb][m][tb] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, xb[tb][i][0], acc[rb][m][tb], 0, 0, 0);
                        acc[rb][m][tb] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, xb[tb][i][1], acc[rb][m][tb], 0, 0, 0);
                    }
                }
    }

#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) red[wave][rb][m][tb][lane] = acc[rb][m][tb];
    __syncthreads();
    // wave rb < RB finishes row block rb
    if (wave >= RB) return;
    const int rb = wave;
    f32x4_t fin[NMAT][TB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            f32x4_t v = red[0][rb][m][tb][lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                const f32x4_t u = red[w][rb][m][tb][lane];
                v[0] += u[0];
                v[1] += u[1];
                v[2] += u[2];
                v[3] += u[3];
            }
            fin[m][tb] = v;
        }
    // 16x16 MFMA result: lane holds token (lane % 16) of the token block and
    // weight rows 4 * (lane / 16) + r, r = 0..3, of the row block.
    const int orow0 = row0 + rb * 16 + 4 * lq;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int tok = tb * 16 + lr;
        if (orow0 >= rows) continue;
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = orow0 + r;
            if (kDual) {
                const float g = round_bf16(s0[rr] * fin[0][tb][r]);
                const float u = round_bf16(s1[rr] * fin[NMAT - 1][tb][r]);
                o[r] = silu_mul(g, u);
            } else {
                o[r] = s0[rr] * fin[0][tb][r];
            }
        }
        uint2 v;
        v.x = pack_bf16x2(o[0], o[1]);
        v.y = pack_bf16x2(o[2], o[3]);
        if (kPacked && kDual) {
            // h in fragment order for the down pass, every token of the block
            // (zero past M, whose activations are zero): features orow0 .. + 3
            // are four consecutive values of one lane's fragment
            const int k = orow0;  // a multiple of 4
            const int64_t off = (int64_t)tb * 16 * rows + (int64_t)(2 * (k / 64) + (k % 16) / 8) * 512 +
                                (lr + 16 * ((k % 64) / 16)) * 8 + (k % 8);
            *reinterpret_cast<uint2*>(hp + off) = v;
        }
        if (tok < M) *reinterpret_cast<uint2*>(out + (int64_t)tok * rows + orow0) = v;
    }
}

// Largest K whose 16-token activations the dual pass keeps in LDS (128 KiB).
constexpr int kLdsDualMaxK = 4096;

// The packed decode for up to 16 tokens, as three launches that keep every
// CU streaming weights from HBM.  Both streaming kernels keep two register
// buffers of kU KiB pieces per matrix and alternate between them (the loop is
// unrolled by two): the loads of the next group are issued before the current
// group is multiplied, and no buffer is ever copied to another (a copy would
// wait for the loads in flight).  Every load is issued unconditionally: a
// piece past the end loads an in-bounds piece again (a cache hit) and is not
// multiplied, so the compiler's waits count exactly the younger loads.
//
// decode_dual_wave_kernel: the dual pass, persistent (one workgroup of kWaves
// waves per CU).  Each wave owns whole row blocks: it streams the block's
// gate and up codes front to back and runs the block's epilogue itself, so
// no wave waits for another.  Row blocks are dealt to the workgroups first
// (block b goes to workgroup b % G, wave b / G % kWaves), so the CUs differ
// by at most one busy wave.  Every wave walks its block's groups in K order:
// in the piece-major layout the waves, moving at about the same pace, then
// read neighbouring KiBs at any moment, a sweep through the matrix rather
// than a thousand scattered streams (3-5% faster than starting each block at
// its own group on block-major pieces).  The sums depend only on kU, not on
// the grid.  The activations' B operands come
// either from a copy of x in LDS in fragment order, made by the workgroup
// before its first item (kXLds), or from global memory with every item's
// weights (two 16-byte loads per piece and lane, rows past M read as
// zeros): the copy costs every CU the whole of x before it can start (about
// 3.6 us at 16 tokens of 3584), the per-item loads cost L1 and L2 traffic in
// proportion to the tokens; at the Qwen2-7B shape the loads are faster up to
// 14 tokens (0.6-1.4 us at 13 and 14) and the copy 0.7-1.3 us faster at 16.
// K % 128 == 0,
// rows % 16 == 0, M <= 16; with kXLds K <= kLdsDualMaxK.
template <int kU, bool kXLds>
struct DualBuf {
    uint4 w[2][kU];
    uint4 x[kXLds ? 1 : kU][2];  // the activations' fragments 2p, 2p + 1 of piece p (not kXLds)
    float sg[4], su[4];          // the row scales of the item's block (this lane's rows)
};

template <int kWaves, int kU, bool kXLds>
__global__ __launch_bounds__(64 * kWaves) void decode_dual_wave_kernel(
    uint16_t* __restrict__ out, uint16_t* __restrict__ hp, const uint16_t* __restrict__ x,
    const uint8_t* __restrict__ w0, const float* __restrict__ s0, const uint8_t* __restrict__ w1,
    const float* __restrict__ s1, int M, int K, int rows) {
    __shared__ uint4 xs[kXLds ? kLdsDualMaxK / 32 * 64 : 1];  // fragment f, lane l: piece 64 f + l
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: loop bounds stay scalar
    const int lr = lane & 15, lq = lane >> 4;
    const int nblocks = rows / 16;
    const int npieces = K / 64;                  // 1-KiB pieces per row block and matrix
    const int ngroups = (npieces + kU - 1) / kU;
    const int G = gridDim.x;
    const int stride = kWaves * G;
    const int b0 = wave * G + blockIdx.x;
    const int nb = b0 < nblocks ? (nblocks - 1 - b0) / stride + 1 : 0;
    const int nit = nb * ngroups;  // (block, group) items of this wave
    // item it: block b0 + (it / ngroups) stride, group it % ngroups
    auto item_group = [&](int it, int& b) {
        b = b0 + (it / ngroups) * stride;
        return it % ngroups;
    };
    auto load_item = [&](int it, DualBuf<kU, kXLds>& q) {
        int b;
        const int g = item_group(it, b);
        // piece p of block b: KiB p * nblocks + b (the ABI keeps rows * K below 2^31)
        const uint32_t bytes = (uint32_t)rows * (uint32_t)K;
        const __amdgpu_buffer_rsrc_t r0 = rsrc_of(w0, bytes);
        const __amdgpu_buffer_rsrc_t r1 = rsrc_of(w1, bytes);
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const uint32_t so = ((uint32_t)min(g * kU + i, npieces - 1) * (uint32_t)nblocks + (uint32_t)b) * 1024u;
            q.w[0][i] = bload16(r0, lane * 16, so);
            q.w[1][i] = bload16(r1, lane * 16, so);
        }
        if (!kXLds) {
            // lane l: token l % 16 (zeros past M through the range check),
            // codes 64 p + 16 (l / 16) + 0..7 and + 8..15
            const __amdgpu_buffer_rsrc_t rx = rsrc_of(x, (uint32_t)(M * K * 2));
#pragma unroll
            for (int i = 0; i < (kXLds ? 1 : kU); ++i) {
                const int pp = min(g * kU + i, npieces - 1);
                const uint32_t xo = lr < M ? (uint32_t)((lr * K + 64 * pp + 16 * lq) * 2) : 0x80000000u;
                q.x[i][0] = bload16(rx, xo, 0);
                q.x[i][1] = bload16(rx, xo + 16u, 0);
            }
        }
        const uint4 vg = bload16(rsrc_of(s0 + b * 16, 64), lq * 16, 0);
        const uint4 vu = bload16(rsrc_of(s1 + b * 16, 64), lq * 16, 0);
        q.sg[0] = __uint_as_float(vg.x), q.sg[1] = __uint_as_float(vg.y);
        q.sg[2] = __uint_as_float(vg.z), q.sg[3] = __uint_as_float(vg.w);
        q.su[0] = __uint_as_float(vu.x), q.su[1] = __uint_as_float(vu.y);
        q.su[2] = __uint_as_float(vu.z), q.su[3] = __uint_as_float(vu.w);
    };
    f32x4_t acc[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
    auto run_item = [&](int it, const DualBuf<kU, kXLds>& q) {
        int b;
        const int g = item_group(it, b);
        if (it % ngroups == 0) {
            acc[0] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            acc[1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int p = g * kU + i;
            if (p < npieces) {
                const bf16x8_t xb0 = __builtin_bit_cast(bf16x8_t, kXLds ? xs[(2 * p) * 64 + lane] : q.x[i][0]);
                const bf16x8_t xb1 =
                    __builtin_bit_cast(bf16x8_t, kXLds ? xs[(2 * p + 1) * 64 + lane] : q.x[i][kXLds ? 0 : 1]);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(q.w[m][i].x, q.w[m][i].y), xb0,
                                                                    acc[m], 0, 0, 0);
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(q.w[m][i].z, q.w[m][i].w), xb1,
                                                                    acc[m], 0, 0, 0);
                }
            }
        }
        if (it % ngroups == ngroups - 1) {
            // lane: token lr, rows orow0 .. + 3 of block b
            const int orow0 = b * 16 + 4 * lq;
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[r] = silu_mul(round_bf16(q.sg[r] * acc[0][r]), round_bf16(q.su[r] * acc[1][r]));
            uint2 v;
            v.x = pack_bf16x2(o[0], o[1]);
            v.y = pack_bf16x2(o[2], o[3]);
            const int k = orow0;  // h in fragment order for the down pass (token block 0)
            const int64_t off =
                (int64_t)(2 * (k / 64) + (k % 16) / 8) * 512 + (lr + 16 * ((k % 64) / 16)) * 8 + (k % 8);
            *reinterpret_cast<uint2*>(hp + off) = v;
            if (lr < M) *reinterpret_cast<uint2*>(out + (int64_t)lr * rows + orow0) = v;
        }
    };
    DualBuf<kU, kXLds> qa, qb;
    if (nit > 0) load_item(0, qa);
    // x into LDS while the first loads are in flight (every load of the copy
    // issued before the first LDS write)
    if (kXLds) {
        const int pieces = K / 32 * 64;
        constexpr int kPer = kLdsDualMaxK / 32 * 64 / (64 * kWaves);
        uint4 v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int p = threadIdx.x + j * 64 * kWaves;
            const int l = p & 63, f = p >> 6;
            const int k0 = 64 * (f >> 1) + 16 * (l >> 4) + 8 * (f & 1);
            v[j] = p < pieces && (l & 15) < M ? *reinterpret_cast<const uint4*>(x + (int64_t)(l & 15) * K + k0)
                                              : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int p = threadIdx.x + j * 64 * kWaves;
            if (p < pieces) xs[p] = v[j];
        }
        __syncthreads();
    }
    for (int it = 0; it < nit; it += 2) {
        load_item(min(it + 1, nit - 1), qb);
        run_item(it, qa);
        if (it + 1 >= nit) break;
        load_item(min(it + 2, nit - 1), qa);
        run_item(it + 1, qb);
    }
}

// decode_down_split_kernel: the down pass split along K.  Workgroup
// (group, s), s = blockIdx.x % S, multiplies the 8 row blocks 8 group .. + 7
// (one per wave) by the s-th of S slices of h: it first copies the slice of
// the fragment-order h (2 KiB per 64-code piece, at most kDownMaxSlice pieces)
// into LDS, then each wave streams its block's codes of the slice (kU KiB
// pieces per group, two buffers as above) and writes its fp32 sums, 16 tokens
// x 16 rows, to part[s][token][row].  Only weights stream from HBM: each slice
// of h is read from L2 once per workgroup instead of once per row block.
// decode_down_reduce_kernel then adds the S partial sums of each output in
// slice order and applies the row scale; S depends on the shape alone, so the
// result does not depend on the device.  K % 64 == 0, rows % 128 == 0.
constexpr int kDownMaxSlice = 64;  // 64-code pieces of h per slice (128 KiB of LDS)
template <int kU>
__global__ __launch_bounds__(512) void decode_down_split_kernel(float* __restrict__ part,
                                                                const uint16_t* __restrict__ hp,
                                                                const uint8_t* __restrict__ w, int K, int rows,
                                                                int S) {
    __shared__ uint4 hs[kDownMaxSlice * 128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const int s = blockIdx.x % S, grp = blockIdx.x / S;
    const int npieces = K / 64;
    const int p0 = (int)((int64_t)s * npieces / S), p1 = (int)((int64_t)(s + 1) * npieces / S);
    const int np = p1 - p0;  // 1 .. kDownMaxSlice
    const int ngroups = (np + kU - 1) / kU;
    const int rb = grp * 8 + wave;
    const __amdgpu_buffer_rsrc_t wr = rsrc_of(w, (uint32_t)rows * (uint32_t)K);  // piece p of block rb: KiB p * rows / 16 + rb
    auto load_group = [&](int g, uint4 (&wq)[kU]) {
#pragma unroll
        for (int i = 0; i < kU; ++i) wq[i] = bload16(wr, lane * 16,
                                      ((uint32_t)(p0 + min(g * kU + i, np - 1)) * (uint32_t)(rows / 16) + (uint32_t)rb) * 1024u);
    };
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto run_group = [&](int g, const uint4 (&wq)[kU]) {
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int p = g * kU + i;
            if (p < np) {
                const bf16x8_t h0 = __builtin_bit_cast(bf16x8_t, hs[(2 * p) * 64 + lane]);
                const bf16x8_t h1 = __builtin_bit_cast(bf16x8_t, hs[(2 * p + 1) * 64 + lane]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(wq[i].x, wq[i].y), h0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(wq[i].z, wq[i].w), h1, acc, 0, 0, 0);
            }
        }
    };
    uint4 wa[kU], wbuf[kU];
    load_group(0, wa);
    {
        // the slice: fragments 2 p0 .. 2 p1 - 1, 64 pieces of 16 bytes each
        const uint4* src = reinterpret_cast<const uint4*>(hp) + (int64_t)p0 * 128;
        constexpr int kPer = kDownMaxSlice * 128 / 512;
        uint4 v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + j * 512;
            v[j] = i < np * 128 ? src[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + j * 512;
            if (i < np * 128) hs[i] = v[j];
        }
    }
    __syncthreads();
    for (int g = 0; g < ngroups; g += 2) {
        load_group(min(g + 1, ngroups - 1), wbuf);
        run_group(g, wa);
        if (g + 1 >= ngroups) break;
        load_group(min(g + 2, ngroups - 1), wa);
        run_group(g + 1, wbuf);
    }
    // lane: token lr, rows rb * 16 + 4 lq .. + 3
    *reinterpret_cast<f32x4_t*>(part + ((int64_t)s * 16 + lr) * rows + rb * 16 + 4 * lq) = acc;
}

// out[m, c] = bf16(sd[c] * (part[0][m][c] + part[1][m][c] + ... + part[S-1][m][c])), m < M;
// one thread per four consecutive outputs, the partial sums loaded eight
// slices at a time (all eight loads in flight before the first add) and added
// in slice order.
__global__ __launch_bounds__(256) void decode_down_reduce_kernel(uint16_t* __restrict__ out,
                                                                 const float* __restrict__ part,
                                                                 const float* __restrict__ sd, int M, int rows,
                                                                 int S) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int q = rows / 4;
    if (t >= M * q) return;
    const int m = t / q, c = (t - m * q) * 4;
    f32x4_t a = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < S; s0 += 8) {
        f32x4_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = *reinterpret_cast<const f32x4_t*>(part + ((int64_t)min(s0 + j, S - 1) * 16 + m) * rows + c);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (s0 + j >= S) break;
            if (s0 + j == 0) {
                a = v[0];
            } else {
                a[0] += v[j][0];
                a[1] += v[j][1];
                a[2] += v[j][2];
                a[3] += v[j][3];
            }
        }
    }
    uint2 o;
    o.x = pack_bf16x2(sd[c] * a[0], sd[c + 1] * a[1]);
    o.y = pack_bf16x2(sd[c + 2] * a[2], sd[c + 3] * a[3]);
    *reinterpret_cast<uint2*>(out + (int64_t)m * rows + c) = o;
}

// Slices of the split down pass for rows = C, K = H: enough workgroups (8 row
// blocks each) for a 256-CU device, no slice longer than kDownMaxSlice pieces
// and none empty.  A function of the shape alone.
static int down_slices(int rows, int K) {
    const int groups = rows / 128;
    const int npieces = K / 64;
    int S = 256 / groups;
    const int min_s = (npieces + kDownMaxSlice - 1) / kDownMaxSlice;
    if (S < min_s) S = min_s;
    if (S > npieces) S = npieces;
    return S < 1 ? 1 : S;
}

// Few-token form (M <= 4) of the passes, on the vector ALU.  With one to
// four tokens the MFMA above multiplies mostly zero columns and spends as many
// load instructions on activations as on weights.  Here the 64 lanes of a wave
// split K instead: one load instruction reads 1 KiB of one weight row (lane l:
// bytes [1024 w + 16 l, +16)), full cache lines in order, and the matching
// activations of each token, loaded once per 1 KiB window, serve all R rows
// (NMAT * R row streams) of the wave.  Products accumulate two at a time with
// v_dot2c_f32_bf16 on packed bf16 pairs (the e4m3 weights widened exactly to
// bf16), so neither operand is unpacked to fp32: at four tokens the unpacking
// and one FMA per element per token would otherwise make the pass VALU-bound.
// Each lane keeps fp32 partial sums per (row, token); one cross-lane sum per
// (row, token) at the end.  Every (row, token) sum sees the same sequence of
// dot2 steps whatever R and U are, so the passes below agree bit for bit with
// each other on the same rows.
//   kSmallDualSilu : g, u rows of w0, w1 -> out[t, row] = bf16(silu(bf16(s0 g)) * bf16(s1 u))
//   kSmallDualGU   : g, u rows of w0, w1 -> out[t, row] = bf16(s0 g), out[t, rows + row] = bf16(s1 u)
//   kSmallSingle   : rows of w0 -> out[t, row] = bf16(s0 y), activations x[t, k]
//   kSmallSingleSiluIn: the same with activations bf16(silu(g) * u) formed on
//                    the fly from g = x[t, k], u = x[t, K + k] (the fused
//                    SiLU-input down projection: the product is recomputed by
//                    every wave that needs it)
// kBf16W: bf16 weights without scales (8 per 16-byte load, 512 K per window).
// U windows of loads are issued before any is used.  kKS > 1 splits each row's
// windows over kKS waves of the workgroup (part p takes windows p, p + kKS,
// ...: an order that depends on kKS alone, not on R or U); the parts' sums
// meet in LDS and are added in part order.  Long rows (the down projection)
// then keep more bytes in flight.  out_ld / x_ld: row strides in elements.
enum : int { kSmallDualSilu = 0, kSmallDualGU = 1, kSmallSingle = 2, kSmallSingleSiluIn = 3 };

template <int kMode, bool kBf16W, int MT, int R, int U, int kWaves, int kKS>
__global__ __launch_bounds__(64 * kWaves) void gemv_small_kernel(
    uint16_t* __restrict__ out, int out_ld, const uint16_t* __restrict__ x, int x_ld,
    const uint8_t* __restrict__ w0, const float* __restrict__ s0, const uint8_t* __restrict__ w1,
    const float* __restrict__ s1, int M, int K, int rows) {
    constexpr bool kDual = kMode == kSmallDualSilu || kMode == kSmallDualGU;
    constexpr bool kSiluIn = kMode == kSmallSingleSiluIn;
    constexpr int NMAT = kDual ? 2 : 1;
    constexpr int kWB = kBf16W ? 2 : 1;   // weight bytes per element
    constexpr int kEPL = 16 / kWB;        // elements per lane per window (one 16-byte load)
    constexpr int kWin = 64 * kEPL;       // elements per window
    constexpr int kXL = kEPL / 8;         // 16-byte activation loads per token per window (x2 for g and u)
    static_assert(kWaves % kKS == 0, "whole groups of waves per row set");
    constexpr int kGroups = kWaves / kKS;
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int part = wid % kKS;
    const int row0 = (blockIdx.x * kGroups + wid / kKS) * R;  // rows % R == 0
    // (with kKS > 1 every wave reaches the barrier below; a wave past the
    // last row reads row 0 and stores nothing)
    if (kKS == 1 && row0 >= rows) return;
    const bool valid = row0 < rows;
    const int rowa = valid ? row0 : 0;
    const uint8_t* wr[R][NMAT];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        wr[r][0] = w0 + (int64_t)(rowa + r) * K * kWB;
        if (kDual) wr[r][NMAT - 1] = w1 + (int64_t)(rowa + r) * K * kWB;
    }
    float acc[R][NMAT][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[r][m][t] = 0.0f;

    const int nwin = (K + kWin - 1) / kWin;
    for (int i = 0; i * kKS + part < nwin; i += U) {
        uint4 wv[U][R][NMAT], xv[U][MT][kSiluIn ? 2 : 1][kXL];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // past the row end (a partial last window, or a window past the
            // last): load the row's last 16 bytes, and zero the activations
            const int k = ((i + u) * kKS + part) * kWin + lane * kEPL;
            ok[u] = k < K;
            const int kc = ok[u] ? k : K - kEPL;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) wv[u][r][m] = *reinterpret_cast<const uint4*>(wr[r][m] + kc * kWB);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const uint16_t* xt = x + (int64_t)min(t, M - 1) * x_ld + kc;
#pragma unroll
                for (int p = 0; p < (kSiluIn ? 2 : 1); ++p)
#pragma unroll
                    for (int c = 0; c < kXL; ++c)
                        xv[u][t][p][c] = *reinterpret_cast<const uint4*>(xt + p * K + 8 * c);
            }
        }
        // every load of the U windows is in flight before the first use (the
        // compiler would otherwise trade them for registers one at a time)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // activations stay packed bf16 pairs (zero past the row end or the
            // last token); the fused SiLU input rounds silu(g) * u to bf16 first
            uint32_t xp[MT][kEPL / 2];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const bool use = ok[u] && t < M;
#pragma unroll
                for (int c = 0; c < kXL; ++c) {
                    const uint32_t* q = reinterpret_cast<const uint32_t*>(&xv[u][t][0][c]);
                    const uint32_t* qu = reinterpret_cast<const uint32_t*>(&xv[u][t][kSiluIn ? 1 : 0][c]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t v = q[e];
                        if (kSiluIn)
                            v = pack_bf16x2(silu_mul(bf16lo(q[e]), bf16lo(qu[e])), silu_mul(bf16hi(q[e]), bf16hi(qu[e])));
                        xp[t][4 * c + e] = use ? v : 0u;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    // weights as bf16 pairs: e4m3 widens exactly (every e4m3
                    // value is a bf16 value)
                    const uint32_t* q = reinterpret_cast<const uint32_t*>(&wv[u][r][m]);
                    uint32_t wp[kEPL / 2];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (kBf16W) {
                            wp[e] = q[e];
                        } else {
                            wp[2 * e] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16(q[e], false));
                            wp[2 * e + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16(q[e], true));
                        }
                    }
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        float a = acc[r][m][t];
#pragma unroll
                        for (int j = 0; j < kEPL / 2; ++j) a = dot2_bf16(wp[j], xp[t][j], a);
                        acc[r][m][t] = a;
                    }
                }
        }
    }
    // lane 0 finishes the rows
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[r][m][t] = wave_sum(acc[r][m][t]);
    if (kKS > 1) {
        __shared__ float part_sum[kWaves][R * NMAT * MT];
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int t = 0; t < MT; ++t) part_sum[wid][(r * NMAT + m) * MT + t] = acc[r][m][t];
        }
        __syncthreads();
        if (part != 0) return;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    float v = part_sum[wid][(r * NMAT + m) * MT + t];
#pragma unroll
                    for (int p = 1; p < kKS; ++p) v += part_sum[wid + p][(r * NMAT + m) * MT + t];
                    acc[r][m][t] = v;
                }
    }
    if (lane != 0 || !valid) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        const float sa = kBf16W ? 1.0f : s0[row];
        const float sb = (kBf16W || !kDual) ? 1.0f : s1[row];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t >= M) continue;
            uint16_t* o = out + (int64_t)t * out_ld;
            if (kMode == kSmallDualSilu) {
                const float g = round_bf16(sa * acc[r][0][t]);
                const float u = round_bf16(sb * acc[r][NMAT - 1][t]);
                o[row] = (uint16_t)(pack_bf16x2(silu_mul(g, u), 0.0f) & 0xffffu);
            } else if (kMode == kSmallDualGU) {
                o[row] = (uint16_t)(pack_bf16x2(sa * acc[r][0][t], 0.0f) & 0xffffu);
                o[rows + row] = (uint16_t)(pack_bf16x2(sb * acc[r][NMAT - 1][t], 0.0f) & 0xffffu);
            } else {
                o[row] = (uint16_t)(pack_bf16x2(sa * acc[r][0][t], 0.0f) & 0xffffu);
            }
        }
    }
}

// Rows per wave (R), windows in flight per wave (U) and waves per row (KS) of
// a few-token pass, by weight type, projection (kDownW: the down
// projection's weights) and token count.  Each
// row group is split over KS waves of one workgroup; a workgroup holds
// max(4, KS) waves.  Measured with C = 4096, H = 14336 and the weights
// streamed from HBM:
//  * e4m3, one token: the down projection's long rows ran at 4.8 TB/s as one
//    wave per two rows (12.3 us) and at 5.05 TB/s as four rows over eight
//    waves (11.6 us): each activation load then serves four rows and each
//    wave's walk is short; one row per wave, or sixteen, ran slower.  The
//    gate/up pass, one row over two waves with two windows in flight each,
//    took the call from 32.1-32.4 to 31.9 us (two rows over four waves: 1%
//    less; four or eight waves per row, or four rows per wave: slower).
//  * e4m3, two tokens: one gate/up row and four windows in flight per wave,
//    two down rows with two windows, no split (the one-token split: 1% slower).
//  * e4m3, three and four tokens: the activation loads outnumber the weight
//    loads; two rows per wave share each, one window in flight, no split (the
//    one-token split took four tokens from 50 to 60 us).
//  * bf16 rows (twice the windows of e4m3 rows) split over four waves in both
//    projections (the single-token bf16 decode 64 -> 60 us); four down rows
//    per wave at four tokens (74 -> 69 us).
// More loads in flight per wave than these ran slower.  KS fixes the order of
// every (row, token) sum (part p sums windows p, p + KS, ...; the parts are
// added in part order) and R and U do not: at a given token count every arm
// sums each projection alike, bit for bit.
struct SmallCfg {
    int R, U, KS;
};
template <bool kBf16W, bool kDownW, int MT>
constexpr SmallCfg small_cfg() {
    constexpr bool kWide = MT > 2;
    if (kBf16W) return kDownW ? SmallCfg{kWide ? 4 : 2, kWide ? 1 : 2, 4} : SmallCfg{kWide ? 2 : 1, kWide ? 1 : 4, 4};
    if (kWide) return SmallCfg{2, 1, 1};
    if (MT == 2) return kDownW ? SmallCfg{2, 2, 1} : SmallCfg{1, 4, 1};
    return kDownW ? SmallCfg{4, 2, 8} : SmallCfg{1, 2, 2};
}
constexpr int kSmallMinWaves = 4;

template <int kMode, bool kBf16W, int MT, bool kDownW>
static hipError_t small_pass(uint16_t* out, int out_ld, const uint16_t* x, int x_ld, const uint8_t* w0,
                             const float* s0, const uint8_t* w1, const float* s1, int M, int K, int rows,
                             hipStream_t s) {
    constexpr SmallCfg cfg = small_cfg<kBf16W, kDownW, MT>();
    constexpr int kW = cfg.KS > kSmallMinWaves ? cfg.KS : kSmallMinWaves;  // waves per workgroup
    constexpr int G = kW / cfg.KS;                                         // row groups per workgroup
    const int groups = rows / cfg.R;  // rows are multiples of 128: whole row groups
    hipLaunchKernelGGL((gemv_small_kernel<kMode, kBf16W, MT, cfg.R, cfg.U, kW, cfg.KS>), dim3((groups + G - 1) / G),
                       dim3(64 * kW), 0, s, out, out_ld, x, x_ld, w0, s0, w1, s1, M, K, rows);
    return hipGetLastError();
}

// The three arms of the few-token decode (gu: [M, 2H] workspace of the
// non-split arms).
template <bool kBf16W, int MT>
static hipError_t launch_decode_small(uint16_t* out, uint16_t* h, uint16_t* gu, const uint16_t* x,
                                      const uint8_t* wg, const float* sg, const uint8_t* wu, const float* su,
                                      const uint8_t* wd, const float* sd, int arm, int M, int C, int H,
                                      hipStream_t s) {
    hipError_t e;
    switch (arm) {
        case kDecodeSiluInput:
            e = small_pass<kSmallDualGU, kBf16W, MT, false>(gu, 2 * H, x, C, wg, sg, wu, su, M, C, H, s);
            if (e != hipSuccess) return e;
            return small_pass<kSmallSingleSiluIn, kBf16W, MT, true>(out, C, gu, 2 * H, wd, sd, nullptr, nullptr, M, H,
                                                              C, s);
        case kDecodePerProjection:
            e = small_pass<kSmallSingle, kBf16W, MT, false>(gu, 2 * H, x, C, wg, sg, nullptr, nullptr, M, C, H, s);
            if (e != hipSuccess) return e;
            e = small_pass<kSmallSingle, kBf16W, MT, false>(gu + H, 2 * H, x, C, wu, su, nullptr, nullptr, M, C, H, s);
            if (e != hipSuccess) return e;
            e = launch_swiglu(h, nullptr, gu, M, H, s);
            if (e != hipSuccess) return e;
            return small_pass<kSmallSingle, kBf16W, MT, true>(out, C, h, H, wd, sd, nullptr, nullptr, M, H, C, s);
        default:
            e = small_pass<kSmallDualSilu, kBf16W, MT, false>(h, H, x, C, wg, sg, wu, su, M, C, H, s);
            if (e != hipSuccess) return e;
            return small_pass<kSmallSingle, kBf16W, MT, true>(out, C, h, H, wd, sd, nullptr, nullptr, M, H, C, s);
    }
}

template <bool kBf16W>
static hipError_t launch_decode_small_m(uint16_t* out, uint16_t* h, uint16_t* gu, const uint16_t* x,
                                        const uint8_t* wg, const float* sg, const uint8_t* wu, const float* su,
                                        const uint8_t* wd, const float* sd, int arm, int M, int C, int H,
                                        hipStream_t s) {
    if (M == 1) return launch_decode_small<kBf16W, 1>(out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H, s);
    if (M == 2) return launch_decode_small<kBf16W, 2>(out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H, s);
    if (M == 3) return launch_decode_small<kBf16W, 3>(out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H, s);
    return launch_decode_small<kBf16W, 4>(out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H, s);
}

template <int TB, int RB_DUAL>
static hipError_t launch_decode_tb(uint16_t* out, uint16_t* h, const uint16_t* x, const uint8_t* wg,
                                   const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd,
                                   const float* sd, int M, int C, int H, hipStream_t s) {
    // H and C are multiples of 128, so whole row blocks always
    hipLaunchKernelGGL((decode_kernel<true, TB, RB_DUAL, kDualWaves>), dim3(H / (16 * RB_DUAL)),
                       dim3(64 * kDualWaves), 0, s, h, nullptr, x, wg, sg, wu, su, M, C, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_kernel<false, TB, 1, kDownWaves>), dim3(C / 16), dim3(64 * kDownWaves), 0, s, out,
                       nullptr, h, wd, sd, nullptr, nullptr, M, H, C);
    return hipGetLastError();
}

hipError_t launch_decode(uint16_t* out, uint16_t* h, uint16_t* gu, const uint16_t* x, const uint8_t* wg,
                         const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd, const float* sd,
                         int arm, bool bf16_weights, int M, int C, int H, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (bf16_weights)
        return launch_decode_small_m<true>(out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H, s);
    if (M <= 4) return launch_decode_small_m<false>(out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H, s);
    if (M <= 16) return launch_decode_tb<1, kDualRB>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
    return launch_decode_tb<2, kDualRB>(out, h, x, wg, sg, wu, su, wd, sd, M, C, H, s);
}

// The packed decode layout of an e4m3 weight [rows, cols] (rows % 16 == 0,
// cols % 64 == 0): 16-byte piece p of the output = lane l = p % 64 of 1 KiB
// block b = p / 64; block b = (64-code chunk kc, row block rb), b = kc * rows /
// 16 + rb (piece-major); the piece is row 16 rb + l % 16, codes 64 kc +
// 16 (l / 16) .. + 15.  Thread t reads piece t of the block-major order and
// writes it where the layout puts it.
__global__ __launch_bounds__(256) void pack_weight_kernel(uint8_t* __restrict__ dst, const uint8_t* __restrict__ w,
                                                          int64_t pieces, int cols) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= pieces) return;
    const int l = (int)(p % 64);
    const int64_t b = p / 64;
    const int kcs = cols / 64;
    const int64_t rb = b / kcs;
    const int kc = (int)(b % kcs);
    const uint8_t* src = w + (rb * 16 + l % 16) * cols + kc * 64 + 16 * (l / 16);
    const int64_t bp = (int64_t)kc * (pieces / 64 / kcs) + rb;  // pieces / 64 / kcs = rows / 16
    *reinterpret_cast<uint4*>(dst + (bp * 64 + l) * 16) = *reinterpret_cast<const uint4*>(src);
}

hipError_t launch_pack_weight(uint8_t* dst, const uint8_t* w, int64_t rows, int cols, hipStream_t s) {
    const int64_t pieces = rows * cols / 16;
    if (pieces == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, dst, w, pieces,
                       cols);
    return hipGetLastError();
}

// x [M, K] bf16 -> fragment order for TB token blocks (see decode_kernel's
// kPacked), zero for tokens past M.  One thread per 16-byte piece.
__global__ __launch_bounds__(256) void pack_x_kernel(uint16_t* __restrict__ xp, const uint16_t* __restrict__ x,
                                                     int M, int K, int64_t pieces) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= pieces) return;
    const int l = (int)(p % 64);
    const int64_t fa = p / 64;
    const int nf = K / 32;
    const int tb = (int)(fa / nf), f = (int)(fa % nf);
    const int tok = tb * 16 + l % 16;
    const int k0 = 64 * (f / 2) + 16 * (l / 16) + 8 * (f % 2);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok < M) v = *reinterpret_cast<const uint4*>(x + (int64_t)tok * K + k0);
    *reinterpret_cast<uint4*>(xp + p * 8) = v;
}

// waves per workgroup of the packed passes (timed at M = 16 on the
// Qwen2-7B and Llama-8B shapes over 4, 8 and 16 waves and 1 or 2 chunks in
// flight per wave); the down pass of two token blocks keeps 8 waves, since
// 16 waves of a workgroup have at most 128 registers each
constexpr int kPackedDualWaves = 4;
template <int TB> constexpr int packed_down_waves() { return TB == 1 ? 16 : 8; }

// Workspace of the packed decode, in bf16 elements: x and h in fragment order,
// then (up to 16 tokens) the split down pass's fp32 partial sums.  Never
// smaller for more tokens, so a workspace for the largest batch serves all.
int64_t decode_packed_ws_elems(int M, int C, int H) {
    const int64_t one_block = 16 * ((int64_t)C + H) + 2 * (int64_t)down_slices(C, H) * 16 * C;
    if (M <= 16) return one_block;
    const int64_t two_blocks = 2 * 16 * ((int64_t)C + H);
    return one_block > two_blocks ? one_block : two_blocks;
}

template <int TB>
static hipError_t launch_packed_tb(uint16_t* out, uint16_t* h, uint16_t* xp, uint16_t* hp, const uint8_t* wg,
                                   const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd,
                                   const float* sd, int M, int C, int H, hipStream_t s) {
    hipLaunchKernelGGL((decode_kernel<true, TB, 1, kPackedDualWaves, true>), dim3(H / 16),
                       dim3(64 * kPackedDualWaves), 0, s, h, hp, xp, wg, sg, wu, su, M, C, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kDownW = packed_down_waves<TB>();
    hipLaunchKernelGGL((decode_kernel<false, TB, 1, kDownW, true>), dim3(C / 16), dim3(64 * kDownW), 0, s, out,
                       nullptr, hp, wd, sd, nullptr, nullptr, M, H, C);
    return hipGetLastError();
}

// waves per workgroup and 1-KiB pieces per load group of the 16-token passes
// (the dual pass with x in LDS, and with x loaded per item), and the most
// tokens that load x per item
constexpr int kWaveDualWaves = 8, kWaveDualU = 8, kWaveDualRegU = 2, kDownSplitU = 8;
constexpr int kDualRegMaxM = 14;

hipError_t launch_decode_packed(uint16_t* out, uint16_t* h, uint16_t* ws, const uint16_t* x, const uint8_t* wg,
                                const float* sg, const uint8_t* wu, const float* su, const uint8_t* wd,
                                const float* sd, int M, int C, int H, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipError_t e;
    if (M <= 16) {
        uint16_t* xp = ws;                 // [16 C] fragment order (more than kDualRegMaxM tokens and C > kLdsDualMaxK)
        uint16_t* hp = ws + (int64_t)16 * C;  // [16 H]
        float* part = reinterpret_cast<float*>(ws + (int64_t)16 * (C + H));  // [S][16][C]
        // one persistent workgroup per CU (with x in LDS it fills most of the
        // LDS); the grid size changes only which wave takes a row block, not
        // the sums
        const int grid = min(H / 16, device_cu_count());
        if (M <= kDualRegMaxM) {
            hipLaunchKernelGGL((decode_dual_wave_kernel<kWaveDualWaves, kWaveDualRegU, false>), dim3(grid),
                               dim3(64 * kWaveDualWaves), 0, s, h, hp, x, wg, sg, wu, su, M, C, H);
        } else if (C <= kLdsDualMaxK) {
            hipLaunchKernelGGL((decode_dual_wave_kernel<kWaveDualWaves, kWaveDualU, true>), dim3(grid),
                               dim3(64 * kWaveDualWaves), 0, s, h, hp, x, wg, sg, wu, su, M, C, H);
        } else {
            const int64_t pieces = (int64_t)(C / 32) * 64;
            hipLaunchKernelGGL(pack_x_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, xp, x, M, C,
                               pieces);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((decode_kernel<true, 1, 1, kPackedDualWaves, true>), dim3(H / 16),
                               dim3(64 * kPackedDualWaves), 0, s, h, hp, xp, wg, sg, wu, su, M, C, H);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int S = down_slices(C, H);
        hipLaunchKernelGGL((decode_down_split_kernel<kDownSplitU>), dim3((C / 128) * S), dim3(512), 0, s, part, hp,
                           wd, H, C, S);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int threads = M * (C / 4);
        hipLaunchKernelGGL(decode_down_reduce_kernel, dim3((threads + 255) / 256), dim3(256), 0, s, out, part, sd, M,
                           C, S);
        return hipGetLastError();
    }
    uint16_t* xp = ws;                            // [2][16 C]
    uint16_t* hp = ws + (int64_t)2 * 16 * C;      // [2][16 H]
    const int64_t pieces = (int64_t)2 * (C / 32) * 64;
    hipLaunchKernelGGL(pack_x_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, xp, x, M, C, pieces);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_packed_tb<2>(out, h, xp, hp, wg, sg, wu, su, wd, sd, M, C, H, s);
}

}  // namespace ffn
