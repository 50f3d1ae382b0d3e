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
// A operand, so each lane ends up holding runs of four consecutive output
// features of one token; lane pairs regroup them (v_permlane32_swap) into
// 16-byte stores.  e4m3 weights may meet e5m2 activations (the backward's
// gradients), selected by the MFMA's B-format field.
//
// LDS layout.  Row r of a stage occupies 64 bytes = 4 chunks of 16 bytes;
// chunk c is stored at position c ^ ((r / 4) % 4).  The LDS serves a 16-byte
// read 16 lanes at a time across 64 banks (256 bytes); a fragment read puts 16
// lanes on 16 consecutive rows at one chunk, and the rows that share a bank
// offset (r, r+4, r+8, r+12) land on 4 different positions: no bank
// conflicts.  Global loads put 4 lanes on the 4 chunks of one row.
//
// Pipeline.  K-steps are loaded straight from global memory into a ring of
// five LDS stages (buffer_load_dwordx4 ... lds, no registers), four steps ahead
// of the MFMAs.  The fragments of step k+1 are read from LDS into a second
// register set while the MFMAs of step k run, so a step's MFMAs never wait for
// the LDS; one counted wait (vmcnt) and one barrier per step publish the next
// stage and retire the oldest.  Inside a step the MFMAs, fragment reads and
// global loads are issued in a fixed interleave (the compiler's scheduler is
// fenced off), one MFMA at a time.
//
// Tiled operands.  A load instruction above reads 16 rows x 64 bytes, half of
// sixteen 128-byte lines (the other halves are the next K-step's).  With both
// operands in the tiled layout (common.h, tiled_offset: the 1 KiB each load
// puts into LDS stored contiguously, swizzle included) every load reads eight
// whole lines, one contiguous KiB; the LDS stages, fragment reads and MFMA
// order stay as they are, so the products are bit for bit those of the
// row-major operands.  Only the load offsets change, and the store offsets
// of a SwiGLU output that is itself the down projection's operand (the e4m3
// codes of h, or bf16 h of a bf16 product).
//
// Tile order.  Workgroups are dealt to the 8 XCDs round-robin; the linear id is
// remapped so that each XCD receives a contiguous range of tiles, and inside it
// tiles are grouped 4 weight-panels wide, so the tiles resident on one XCD at a
// time share weight and token panels in that XCD's L2.  The grid is persistent
// (workgroups walk tiles b, b + G, ..., their K-steps one stream across tiles)
// or, on request, one workgroup per tile.
//
// SwiGLU fusion.  With fuse_swiglu the 256 weight rows of a tile are 128 gate
// rows and the 128 matching up rows, arranged so that every wave holds gate and
// up accumulators for the same (token, feature) pairs in matching registers:
// the epilogue rounds g and u to bf16, forms bf16(silu(g) * u), and folds the
// tile's abs-max into one atomic.  Other epilogues: a plain bf16 store; an
// accumulating one (old + product, one rounding: the backward's weight
// gradients); and the SwiGLU backward (dh rounded to bf16, then dgu from dh
// and the forward's gu, with its abs-max).
#include <atomic>

#include "common.h"
#include "launch.h"

namespace ffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

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
constexpr int kTiledStep = 64 * kRowBytes;  // bytes of one K-step of a 64-row group, tiled layout
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
    const float* q_absmax;  // SwiGLU + quantise: the known abs-max of h
    float* q_scale;         // ... and where its dequantisation scale goes
    const uint8_t* aux;     // SwiGLU backward: gu [N, 2H], the layout of out
};

// A buffer resource (V#) for raw byte addressing: base address, no stride,
// num_records bytes; accesses at or beyond num_records read zero and drop
// stores (the range check of buffer instructions).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t num_records) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4_t{(int)(uint32_t)p, (int)(uint32_t)(p >> 32) & 0xffff, (int)num_records, 0x00020000};
}

// One wave-wide direct load: lane l's 16 bytes at rsrc + soff + voff land in
// LDS at lds_addr + 16 l (zeros where the range check fails).  Issued as
// inline assembly so that the compiler does not treat every later LDS read as
// dependent on it (it would otherwise wait for all outstanding loads before
// each read); the kernel orders these loads against its LDS reads itself, with
// counted vmcnt waits and barriers.
__device__ __forceinline__ void load_lds16(uint32_t voff, i32x4_t rsrc, uint32_t soff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
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
    const uint8_t* lds;       // the ring (generic pointer)
    uint32_t lds_wave;        // LDS address of this wave's first load row in stage 0
    uint32_t voff[kLoads];    // byte offset of this lane's row of load i in its wave's 64-row slab
    int a_rd[2], b_rd[2];     // byte offsets of this lane's fragment pieces in a stage
};

// The 64-row slabs of w and x that one wave loads for one tile.
struct TileRsrc {
    i32x4_t a, b;
};

__device__ __forceinline__ void read_frags(Frags& f, const StepIO& io, int g) {
    const uint8_t* st = io.lds + (g % kStages) * kStage;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int blk = (r & 7) >> 1, p = r & 1;
        if (r < 8) f.a[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.a_rd[p] + blk * kBlockBytes);
        else f.b[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.b_rd[p] + blk * kBlockBytes);
    }
}

// Load instruction l (0 .. 2 kLoads - 1; A first) of K-step kk of the tile
// whose slabs are `tr`, into ring slot `stage`.  kTiled: the slabs are in the
// tiled layout, where K-step kk of a 64-row group starts kk * 4 KiB in.
template <bool kTiled>
__device__ __forceinline__ void load_part(const StepIO& io, const TileRsrc& tr, int stage, int kk, int l) {
    const uint32_t kb = (uint32_t)kk * (kTiled ? kTiledStep : kRowBytes);
    const uint32_t st = io.lds_wave + (uint32_t)(stage * kStage);
    if (l < kLoads) load_lds16(io.voff[l], tr.a, kb, st + l * 16 * kRowBytes);
    else load_lds16(io.voff[l - kLoads], tr.b, kb, st + kBM * kRowBytes + (l - kLoads) * 16 * kRowBytes);
}

// The MFMAs of stream step g from `cur`, while the fragments of step g + 1 are
// read into `nxt` and the loads of step g + kAhead (K-step ld_k of the tile
// whose slabs are `tr`) are issued.  The code must be free of branches: the
// scheduling fences order instructions within a basic block only.
// kXBf8: the x fragments (the MFMA's B operand) hold e5m2 codes, selected by
// the instruction's B-format field; the w fragments stay e4m3.
template <bool kFP8, bool kXBf8, bool kTiled>
__device__ __forceinline__ void k_step(f32x16_t (&acc)[4][4], const Frags& cur, Frags& nxt, const GemmArgs& a,
                                       const StepIO& io, int g, const TileRsrc& tr, int ld_k) {
    constexpr int kM = kFP8 ? 16 : 32;  // MFMAs per step
    constexpr int kPerRead = kM / 16, kPerLoad = kM / (2 * kLoads);
    const uint8_t* st = io.lds + ((g + 1) % kStages) * kStage;
    const int ld_stage = (g + kAhead) % kStages;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < kM; ++m) {
        if (m % kPerRead == 0) {
            const int r = m / kPerRead, blk = (r & 7) >> 1, p = r & 1;
            if (r < 8) nxt.a[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.a_rd[p] + blk * kBlockBytes);
            else nxt.b[blk][p] = *reinterpret_cast<const i32x4_t*>(st + io.b_rd[p] + blk * kBlockBytes);
        }
        if (kFP8) {
            const int i = m >> 2, j = m & 3;
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                __builtin_shufflevector(cur.a[i][0], cur.a[i][1], 0, 1, 2, 3, 4, 5, 6, 7),
                __builtin_shufflevector(cur.b[j][0], cur.b[j][1], 0, 1, 2, 3, 4, 5, 6, 7), acc[i][j], 0,
                kXBf8 ? 1 : 0, 0, 127, 0, 127);
        } else {
            const int i = m >> 3, j = (m >> 1) & 3, p = m & 1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cur.a[i][p]),
                                                                __builtin_bit_cast(bf16x8_t, cur.b[j][p]),
                                                                acc[i][j], 0, 0, 0);
        }
        if (m % kPerLoad == kPerLoad - 1) load_part<kTiled>(io, tr, ld_stage, ld_k, m / kPerLoad);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The slabs of w and x that wave `wave` loads for tile t (launch order).
// Weight rows: plain, rows [256 tm + 64 wave, +64) of w; SwiGLU-fused, the
// tile's 128 gate rows [128 tm, +128) of w followed by the matching up rows
// [H + 128 tm, +128), so wave w takes gate rows (w & 1) = 0 or up rows
// (w & 1) = 1, half w >> 1.  Rows past O (plain) and tokens past N are cut
// off by num_records and load as zeros.  Every slab starts at a multiple of
// 64 rows, so in the tiled layout it is one 64-row group at the same byte
// offset; a group with any valid row is read whole (the tiled operands hold
// whole groups), one with none as zeros.
template <bool kFused, bool kTiled>
__device__ __forceinline__ TileRsrc tile_rsrc(const GemmArgs& a, int t, int wave) {
    int tm, tn;
    tile_coords(t, a.tiles_m, a.tiles_n, tm, tn);
    const int64_t kb = a.K_bytes;
    int64_t wrow0, wrows;
    if (kFused) {
        wrow0 = (int64_t)((wave & 1) ? a.H : 0) + (int64_t)tm * 128 + (wave >> 1) * 64;
        wrows = 64;
    } else {
        wrow0 = (int64_t)tm * kBM + wave * 64;
        wrows = min((int64_t)64, max((int64_t)0, (int64_t)a.O - wrow0));
    }
    const int64_t xrow0 = (int64_t)tn * kBN + wave * 64;
    int64_t xrows = min((int64_t)64, max((int64_t)0, a.N - xrow0));
    if (kTiled) {
        wrows = wrows > 0 ? 64 : 0;
        xrows = xrows > 0 ? 64 : 0;
    }
    TileRsrc r;
    r.a = make_rsrc(a.w + wrow0 * kb, (uint32_t)(wrows * kb));
    r.b = make_rsrc(a.x + xrow0 * kb, (uint32_t)(xrows * kb));
    return r;
}

__device__ __forceinline__ TileRsrc select_rsrc(bool c, const TileRsrc& x, const TileRsrc& y) {
    TileRsrc r;
    r.a = c ? x.a : y.a;
    r.b = c ? x.b : y.b;
    return r;
}

// Store instructions per lane in one tile's epilogue (16-byte stores; 8-byte
// stores of e4m3 codes when quantising).
template <bool kFused>
constexpr int epilogue_stores() { return kFused ? 16 : 32; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The 16 accumulators of one MFMA block, copied to ordinary registers right
// here.  Written as assembly so that the compiler cannot gather the copies of
// all 256 accumulators at the start of the epilogue (which would exhaust the
// registers); kHazardPad adds the wait states an accumulator read needs after
// the MFMA that wrote it (the first block read after the K loop).
template <bool kHazardPad>
__device__ __forceinline__ f32x16_t read_acc(const f32x16_t& x) {
    f32x16_t v;
    if (kHazardPad) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    asm volatile(
        "v_accvgpr_read_b32 %0, %16\n\tv_accvgpr_read_b32 %1, %17\n\t"
        "v_accvgpr_read_b32 %2, %18\n\tv_accvgpr_read_b32 %3, %19\n\t"
        "v_accvgpr_read_b32 %4, %20\n\tv_accvgpr_read_b32 %5, %21\n\t"
        "v_accvgpr_read_b32 %6, %22\n\tv_accvgpr_read_b32 %7, %23\n\t"
        "v_accvgpr_read_b32 %8, %24\n\tv_accvgpr_read_b32 %9, %25\n\t"
        "v_accvgpr_read_b32 %10, %26\n\tv_accvgpr_read_b32 %11, %27\n\t"
        "v_accvgpr_read_b32 %12, %28\n\tv_accvgpr_read_b32 %13, %29\n\t"
        "v_accvgpr_read_b32 %14, %30\n\tv_accvgpr_read_b32 %15, %31"
        : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5]), "=v"(v[6]), "=v"(v[7]),
          "=v"(v[8]), "=v"(v[9]), "=v"(v[10]), "=v"(v[11]), "=v"(v[12]), "=v"(v[13]), "=v"(v[14]), "=v"(v[15])
        : "a"(x[0]), "a"(x[1]), "a"(x[2]), "a"(x[3]), "a"(x[4]), "a"(x[5]), "a"(x[6]), "a"(x[7]), "a"(x[8]),
          "a"(x[9]), "a"(x[10]), "a"(x[11]), "a"(x[12]), "a"(x[13]), "a"(x[14]), "a"(x[15]));
    return v;
}

// Lanes l and l + 32 hold the same token row and interleaved runs of four
// features: lane l runs 0 and 2 of each 32-feature block (features 0-3,
// 16-19), lane l + 32 runs 1 and 3 (4-7, ...), as fh * 4 + 8 g.  One
// v_permlane32_swap per dword pair regroups runs 2q and 2q + 1 so that lane l
// holds features 16q + 0..7 and lane l + 32 features 16q + 8..15: one 16-byte
// store each.  x = run 2q, y = run 2q + 1 (two packed dwords each).
__device__ __forceinline__ u32x4_t regroup_runs(uint32_t x0, uint32_t x1, uint32_t y0, uint32_t y1) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    return u32x4_t{s0[0], s1[0], s0[1], s1[1]};
}

// One tile's output.  Every lane issues exactly epilogue_stores() buffer
// stores; rows past N and features past O are dropped by the buffer's range
// check (their offsets point past num_records), so the count of outstanding
// memory operations stays exact for the pipeline's counted waits.  kQuant
// (SwiGLU only): h is rounded to bf16 as always, its abs-max kept, and the
// stored output is e4m3(h * qinv), the codes ffn_quant_absmax would give h
// with that abs-max.  kAccum (plain output only): the epilogue loads the bf16
// values it will overwrite (out of range: zero) and stores bf16(old + acc * s),
// one rounding.  The loads of 32-row block j + 1 are issued before the wait for
// block j's, so each wait overlaps a block's work.  The loads and waits only
// add memory operations after the pipeline's in-flight loads, which keeps its
// counted waits safe (they wait for at least as much).
// kSwiBwd (plain output only): the product is dh, the gradient of the SwiGLU
// output h = silu(g) * u; it is rounded to bf16 as a plain store would round
// it, and instead of dh the epilogue stores dgu [N, 2H] (dg at feature o, du
// at H + o) from gu [N, 2H] (a.aux, same layout; it may be out itself), with
// swiglu_bwd_pair, keeping the running abs-max of the stored dgu.  Its loads
// of g and u are double-buffered by half-blocks of 32 tokens x 64 features.
template <bool kFP8, bool kFused, bool kQuant, bool kAccum, bool kSwiBwd, bool kTiled>
__device__ __forceinline__ void tile_epilogue(f32x16_t (&acc)[4][4], const GemmArgs& a, int t, float s, float qinv,
                                              int wm, int wn, int fr, int fh, float& amax) {
    int tm, tn;
    tile_coords(t, a.tiles_m, a.tiles_n, tm, tn);
    // recomputed per tile: kept out of registers across the K loop
    asm volatile("" : "+v"(fr), "+v"(fh));
    const int64_t n0 = (int64_t)tn * kBN;
    constexpr int kOutElt = kQuant ? 1 : 2;  // bytes per output element
    uint8_t* base = reinterpret_cast<uint8_t*>(a.out) + n0 * a.ld_out * kOutElt;
    // a tiled SwiGLU output (the e4m3 codes of h, or bf16 h of a bf16
    // product: the next GEMM's operand) has the tile's rows as whole 64-row
    // groups from the same byte offset, rows past N skipped by offset (they
    // are not a prefix there); every other output is row-major, its rows past
    // N cut off by the range
    constexpr bool kTiledOut = kTiled && kFused && (kQuant || !kFP8);
    const int64_t rows_left = kTiledOut ? (a.N - n0 + 63) / 64 * 64 : a.N - n0;
    const int64_t rem = rows_left * (int64_t)a.ld_out * kOutElt;
    const uint32_t nrec = (uint32_t)(rem < ((int64_t)1 << 30) ? rem : ((int64_t)1 << 30));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)nrec, 0x00020000);
    const uint32_t row_bytes = (uint32_t)a.ld_out * kOutElt;
    const int r_base = wn * 128 + fr;  // token row within the tile, block j adds 32 j
    if (kSwiBwd) {
        // gu has the layout of dgu: the same offsets from another base
        const __amdgpu_buffer_rsrc_t grs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.aux) + n0 * a.ld_out * 2, 0, (int)nrec,
                                              0x00020000);
        const uint32_t up_off = (uint32_t)a.O * 2;  // u and du: H = O features further on
        // half-block hb = (token block j = hb / 2, feature blocks i = 2 (hb % 2)
        // + 0..1); its group gi = 2 (i % 2) + q: features o .. o + 7
        auto off_of = [&](int hb, int gi) -> uint32_t {
            const int j = hb >> 1, i = 2 * (hb & 1) + (gi >> 1), q = gi & 1;
            const int o = tm * kBM + wm * 128 + i * 32 + 16 * q + 8 * fh;
            return o < a.O ? (uint32_t)(r_base + 32 * j) * row_bytes + (uint32_t)o * 2 : 0x7fffffffu;
        };
        u32x4_t gv[2][4], uv[2][4];
        auto load_hb = [&](int hb, u32x4_t (&gd)[4], u32x4_t (&ud)[4]) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const uint32_t off = off_of(hb, gi);
                gd[gi] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0));
                ud[gi] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(grs, off + up_off, 0, 0));
            }
        };
        load_hb(0, gv[0], uv[0]);
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) {
            // 8 loads and 8 stores per half-block; after half-block hb's loads
            // come hb + 1's loads and (from hb = 1) hb - 1's stores
            if (hb + 1 < 8) load_hb(hb + 1, gv[(hb + 1) & 1], uv[(hb + 1) & 1]);
            if (hb == 0 || hb == 7) wait_vmcnt<8>();
            else wait_vmcnt<16>();
            __builtin_amdgcn_sched_barrier(0);
            const int j = hb >> 1;
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * (hb & 1) + ii;
                const f32x16_t blk = (i == 0 && j == 0) ? read_acc<true>(acc[i][j]) : read_acc<false>(acc[i][j]);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    uint32_t d[4];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int g = 2 * q + h;
                        d[2 * h] = pack_bf16x2(blk[4 * g + 0] * s, blk[4 * g + 1] * s);
                        d[2 * h + 1] = pack_bf16x2(blk[4 * g + 2] * s, blk[4 * g + 3] * s);
                    }
                    const u32x4_t dv = regroup_runs(d[0], d[1], d[2], d[3]);  // dh, features o .. o + 7
                    const int gi = 2 * ii + q;
                    const u32x4_t gg = gv[hb & 1][gi], uu = uv[hb & 1][gi];
                    u32x4_t og, ou;
                    float m = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float g0, u0, g1, u1;
                        swiglu_bwd_pair(bf16lo(dv[e]), bf16lo(gg[e]), bf16lo(uu[e]), g0, u0);
                        swiglu_bwd_pair(bf16hi(dv[e]), bf16hi(gg[e]), bf16hi(uu[e]), g1, u1);
                        og[e] = pack_bf16x2(g0, g1);
                        ou[e] = pack_bf16x2(u0, u1);
                        m = absmax_acc(absmax_acc(m, bf16lo(og[e])), bf16hi(og[e]));
                        m = absmax_acc(absmax_acc(m, bf16lo(ou[e])), bf16hi(ou[e]));
                    }
                    // rows past N (and features past O) have offsets past the
                    // range, so their stores are dropped; they stay out of the
                    // abs-max too (with tiled operands their codes are whatever
                    // the group's padding holds, so dh there need not be zero).
                    // The mask is the sign of off - nrec, all ones in range: no
                    // lane mask, as the scalar registers are all taken here.
                    const uint32_t off = off_of(hb, gi);
                    const uint32_t keep = (uint32_t)((int32_t)(off - nrec) >> 31);
                    // one running maximum, updated in order (left to itself the
                    // compiler regroups the whole chain and runs out of registers)
                    amax = absmax_acc(amax, __uint_as_float(__float_as_uint(m) & keep));
                    asm volatile("" : "+v"(amax));
                    __builtin_amdgcn_raw_buffer_store_b128(og, rsrc, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(ou, rsrc, off + up_off, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    } else if (!kFused) {
        // the previous values of a block's outputs, in the stored (regrouped)
        // order; v_permlane32_swap is its own inverse, so swapping them back
        // gives the accumulator order.  Two blocks' worth, double-buffered.
        u32x4_t oldv[2][4][2];
        auto load_old = [&](int j, u32x4_t (&dst)[4][2]) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int o = tm * kBM + wm * 128 + i * 32 + 16 * q + 8 * fh;
                    const uint32_t off = o < a.O ? (uint32_t)(r_base + 32 * j) * row_bytes + (uint32_t)o * 2
                                                 : 0x7fffffffu;
                    dst[i][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
                }
        };
        if (kAccum) load_old(0, oldv[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4_t (&old)[4][2] = oldv[j & 1];
            if (kAccum) {
                // 8 loads and 8 stores per block; after block j's loads come
                // block j + 1's loads and (from j = 1) block j - 1's stores
                if (j + 1 < 4) load_old(j + 1, oldv[(j + 1) & 1]);
                if (j == 0 || j == 3) wait_vmcnt<8>();
                else wait_vmcnt<16>();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x16_t blk = (i == 0 && j == 0) ? read_acc<true>(acc[i][j]) : read_acc<false>(acc[i][j]);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    float add[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
                    if (kAccum) {
                        const u32x4_t ov = old[i][q];
                        const auto s0 = __builtin_amdgcn_permlane32_swap(ov[0], ov[2], false, false);
                        const auto s1 = __builtin_amdgcn_permlane32_swap(ov[1], ov[3], false, false);
                        const uint32_t od[4] = {s0[0], s1[0], s0[1], s1[1]};  // d[0], d[1], d[2], d[3]
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            add[2 * e] = bf16lo(od[e]);
                            add[2 * e + 1] = bf16hi(od[e]);
                        }
                    }
                    uint32_t d[4];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int g = 2 * q + h;
                        d[2 * h] = pack_bf16x2(blk[4 * g + 0] * s + add[4 * h], blk[4 * g + 1] * s + add[4 * h + 1]);
                        d[2 * h + 1] =
                            pack_bf16x2(blk[4 * g + 2] * s + add[4 * h + 2], blk[4 * g + 3] * s + add[4 * h + 3]);
                    }
                    const u32x4_t v = regroup_runs(d[0], d[1], d[2], d[3]);
                    const int o = tm * kBM + wm * 128 + i * 32 + 16 * q + 8 * fh;
                    const uint32_t off = o < a.O ? (uint32_t)(r_base + 32 * j) * row_bytes + (uint32_t)o * 2
                                                 : 0x7fffffffu;
                    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = n0 + r_base + 32 * j < a.N;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x16_t gb = (i == 0 && j == 0) ? read_acc<true>(acc[i][j]) : read_acc<false>(acc[i][j]);
                const f32x16_t ub = read_acc<false>(acc[i + 2][j]);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    uint32_t d[4];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int g = 2 * q + h;
                        float hv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float gg = round_bf16(gb[4 * g + e] * s);
                            const float uu = round_bf16(ub[4 * g + e] * s);
                            hv[e] = silu_mul(gg, uu);
                        }
                        d[2 * h] = pack_bf16x2(hv[0], hv[1]);
                        d[2 * h + 1] = pack_bf16x2(hv[2], hv[3]);
                    }
                    float m = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        m = absmax_acc(absmax_acc(m, bf16lo(d[e])), bf16hi(d[e]));
                    amax = absmax_acc(amax, ok ? m : 0.0f);
                    const u32x4_t v = regroup_runs(d[0], d[1], d[2], d[3]);
                    const int o = tm * 128 + wm * 64 + i * 32 + 16 * q + 8 * fh;
                    uint32_t off = (uint32_t)(r_base + 32 * j) * row_bytes + (uint32_t)o * kOutElt;
                    if (kTiledOut)  // rows past N skipped by offset
                        off = ok ? (uint32_t)tiled_offset(r_base + 32 * j, (int64_t)o * kOutElt, row_bytes)
                                 : 0x7fffffffu;
                    if (kQuant) {
                        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                        const u32x2_t c = {
                            pack_e4m3x4(bf16lo(v[0]) * qinv, bf16hi(v[0]) * qinv, bf16lo(v[1]) * qinv, bf16hi(v[1]) * qinv),
                            pack_e4m3x4(bf16lo(v[2]) * qinv, bf16hi(v[2]) * qinv, bf16lo(v[3]) * qinv, bf16hi(v[3]) * qinv)};
                        __builtin_amdgcn_raw_buffer_store_b64(c, rsrc, off, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, off, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
}

template <bool kFP8, bool kFused, bool kQuant, bool kAccum, bool kXBf8 = false, bool kSwiBwd = false,
          bool kTiled = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs a) {
    static_assert(kFused || !kQuant, "quantised output is a SwiGLU epilogue");
    static_assert(!(kFused && kAccum), "accumulation is a plain-output epilogue");
    static_assert(kFP8 || !kXBf8, "e5m2 x is an FP8 operand");
    static_assert(!(kSwiBwd && (kFused || kAccum)), "the SwiGLU backward is a plain-output epilogue of its own");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
    static_assert(kStages * kStage <= 160 * 1024, "LDS ring exceeds the 160 KiB of a CU");
    constexpr int kStoreCnt = epilogue_stores<kFused>();
    static_assert(2 * kLoads * (kAhead - 2) + kStoreCnt <= 63, "vmcnt holds at most 63");

    // Persistent: workgroup b takes tiles b, b + G, b + 2G, ... (launch order,
    // mapped to tile coordinates by tile_coords).  Its K-steps form one stream
    // across its tiles, so the ring never drains between tiles: the first
    // steps of the next tile load while the current tile finishes.
    const int T = a.tiles_m * a.tiles_n;
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int KT = a.K_bytes / kRowBytes;  // even: the ABI requires K % 128 == 0 (elements)

    float s = 1.0f;
    if (kFP8) s = (*a.x_scale) * (*a.w_scale);
    float qinv = 1.0f;
    if (kQuant) {
        float qscale;
        scale_pair(*a.q_absmax, qscale, qinv);
        if (blockIdx.x == 0 && threadIdx.x == 0) *a.q_scale = qscale;
    }

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    StepIO io;
    io.lds = lds;
    f32x16_t acc[4][4];
    // ---- global -> LDS.  One wave instruction fills 1 KiB of a stage = 16
    // rows of 64 bytes; lane l lands at (row l/4, slot l%4) and so fetches
    // chunk (l%4) ^ ((row/4)%4) of its row, which realises the XOR swizzle.
    // Wave w fills rows [64 w, 64 w + 64) of both operands.
    const int lrow = lane >> 2;
    const int lch = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
        io.voff[i] = kTiled ? (uint32_t)(i * 1024 + lane * 16)
                            : (uint32_t)(i * 16 + lrow) * (uint32_t)a.K_bytes + (uint32_t)(lch << 4);
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

    // Loads run kAhead K-steps ahead of the MFMAs, so the last steps of a tile
    // load the first steps of the workgroup's next tile.  After its last tile
    // a workgroup keeps loading steps of that tile again: those loads fill
    // stages that are never read and keep every step's load count, and so the
    // counted waits, uniform.  With KT < kAhead the loads would run more than
    // one tile ahead; such problems get one tile per workgroup (G = T), where
    // every load past the tile's own steps is one of these stand-ins.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    TileRsrc tr_cur = tile_rsrc<kFused, kTiled>(a, b, wave_u);
    TileRsrc tr_nxt = tile_rsrc<kFused, kTiled>(a, b + G < T ? b + G : b, wave_u);
    // K-step of the load issued during step kk of a tile (tile-relative
    // kk + kAhead, wrapped into the next tile)
    auto wrap_k = [&](int k) {
        if (k >= KT) k -= KT;
        if (k >= KT) k -= KT;
        return k;
    };

    // Stream step g lives in stage g % 5.  Before the MFMAs of step g, steps
    // g and g + 1 are in LDS and visible to every wave (the fragments of g are
    // in registers) and this wave has issued the loads of steps up to g + 3.
    // During step g it issues the loads of step g + 4 into the stage of step
    // g - 1, whose fragments every wave finished reading before the barrier
    // that closed step g - 1; after step g it waits for its loads of step
    // g + 2 and meets the others at the barrier.  Memory operations complete
    // in issue order, so "the loads of g + 2 have landed" is "at most the
    // operations issued after them are outstanding": the loads of g + 3 and
    // g + 4, plus, in the first two steps of a tile, the stores of the
    // previous tile's epilogue.
#pragma unroll
    for (int g = 0; g < kAhead; ++g) {
        const TileRsrc tr = select_rsrc(g < KT, tr_cur, tr_nxt);
        const int k = g < KT ? g : wrap_k(g);
#pragma unroll
        for (int l = 0; l < 2 * kLoads; ++l) load_part<kTiled>(io, tr, g, k, l);
    }
    // Stand-ins for the stores of a previous tile's epilogue (dropped by the
    // range check: num_records is 0), so that the first tile's first two
    // waits count the same operations as every later tile's.
    {
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, 0, 0x00020000);
#pragma unroll
        for (int i = 0; i < kStoreCnt; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, none, 16 * i, 0, 0);
    }
    constexpr int kWait = 2 * kLoads * (kAhead - 2);
    wait_vmcnt<kWait + kStoreCnt>();
    barrier();
    Frags f0, f1;
    read_frags(f0, io, 0);

    float amax = 0.0f;
    int g = 0;
    for (int c_t = b; c_t < T; c_t += G) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        // the first pair follows the previous tile's epilogue stores
        {
            const bool own = kAhead < KT;
            const TileRsrc tr = select_rsrc(own, tr_cur, tr_nxt);
            const int k0 = own ? kAhead : wrap_k(kAhead);
            const int k1 = own ? kAhead + 1 : wrap_k(kAhead + 1);
            k_step<kFP8, kXBf8, kTiled>(acc, f0, f1, a, io, g, tr, k0);
            wait_vmcnt<kWait + kStoreCnt>();
            barrier();
            k_step<kFP8, kXBf8, kTiled>(acc, f1, f0, a, io, g + 1, tr, k1);
            wait_vmcnt<kWait + kStoreCnt>();
            barrier();
            g += 2;
        }
        for (int kk = 2; kk < KT; kk += 2, g += 2) {
            const bool own = kk + kAhead < KT;
            const TileRsrc tr = select_rsrc(own, tr_cur, tr_nxt);
            const int k0 = own ? kk + kAhead : wrap_k(kk + kAhead);
            k_step<kFP8, kXBf8, kTiled>(acc, f0, f1, a, io, g, tr, k0);
            wait_vmcnt<kWait>();
            barrier();
            k_step<kFP8, kXBf8, kTiled>(acc, f1, f0, a, io, g + 1, tr, k0 + 1);
            wait_vmcnt<kWait>();
            barrier();
        }
        tile_epilogue<kFP8, kFused, kQuant, kAccum, kSwiBwd, kTiled>(acc, a, c_t, s, qinv, wm, wn, fr, fh, amax);
        const int t2 = c_t + 2 * G;
        tr_cur = tr_nxt;
        tr_nxt = tile_rsrc<kFused, kTiled>(a, t2 < T ? t2 : (c_t + G < T ? c_t + G : c_t), wave_u);
    }
    // the loads past the end still write the ring: let them land before the
    // workgroup's LDS is reused or released
    wait_vmcnt<0>();
    if ((kFused || kSwiBwd) && a.absmax) {
        __syncthreads();
        block_absmax_commit(amax, reinterpret_cast<float*>(lds), a.absmax);
    }
}

// The tiled layout of a [rows, row_bytes] operand: thread t writes the
// t-th 16 bytes of the output (whole 64-row groups), read from the row and
// chunk that tiled_offset puts there (zeros past `rows`).
__global__ __launch_bounds__(256) void tile_pack_kernel(uint8_t* __restrict__ out, const uint8_t* __restrict__ in,
                                                        int64_t rows, int64_t row_bytes, int64_t chunks) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < chunks;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t off = t * 16, group_bytes = 64 * row_bytes;
        const int64_t grp = off / group_bytes, in_grp = off - grp * group_bytes;
        const int64_t step = in_grp >> 12;
        const int blk = (int)(in_grp & 4095), l = (blk & 1023) >> 4;
        const int64_t r = 64 * grp + 16 * (blk >> 10) + (l >> 2);
        const int64_t c = 64 * step + 16 * ((l & 3) ^ (l >> 4));
        uint4 v = {0u, 0u, 0u, 0u};
        if (r < rows) v = *reinterpret_cast<const uint4*>(in + r * row_bytes + c);
        *reinterpret_cast<uint4*>(out + off) = v;
    }
}

hipError_t launch_tile_pack(uint8_t* out, const uint8_t* in, int64_t rows, int64_t row_bytes, hipStream_t s) {
    const int64_t chunks = (rows + 63) / 64 * 64 * row_bytes / 16;
    if (chunks == 0) return hipSuccess;
    const int64_t blocks = min((chunks + 255) / 256, (int64_t)65536);
    hipLaunchKernelGGL(tile_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, in, rows, row_bytes, chunks);
    return hipGetLastError();
}

int device_cu_count() {
    // per device, filled on first use; threads that race here store the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of the persistent grid for T tiles: as many rounds of tiles as
// one workgroup per CU needs, dealt over as few workgroups as still finish in
// that many rounds (a multiple of 8, so that tile b and its workgroup b % G sit
// on the same XCD).  The makespan is the same as with one workgroup per CU;
// the CUs left over (64 of 256 for the 448 tiles of a 3584 x 8192 output) stay
// free for work on other streams.
static int persistent_grid(int T) {
    const int cu = device_cu_count();
    if (T <= cu) return T;
    const int rounds = (T + cu - 1) / cu;
    const int g = ((T + rounds - 1) / rounds + 7) / 8 * 8;
    return min(g, cu);
}

// Abs-max of a plain (unfused) GEMM output, when asked for: a separate pass.
// clear_absmax == false (fused epilogues only): the abs-max is max-accumulated
// into the word as found (the caller zeroed it) instead of cleared first.
// q_absmax / q_scale (SwiGLU only, both or neither): store e4m3 codes of h
// under that known abs-max instead of bf16 h, and its scale.  x_e5m2 (fp8,
// plain output): x holds e5m2 codes.  swiglu_gu (plain output, no
// accumulation): the product is dh and out receives dgu [N, 2O] from gu
// [N, 2O] (may be out), with its abs-max in absmax.  tile_grid: one
// workgroup per output tile instead of the persistent grid, so that the
// hardware hands CUs to kernels on other streams as tiles finish (the
// partial last round of one product fills with the tiles of another).
hipError_t launch_gemm(void* out, float* absmax, const void* x, const float* x_scale, const void* w,
                       const float* w_scale, bool fp8, bool fuse_swiglu, int64_t N, int K, int O,
                       hipStream_t s, const float* q_absmax, float* q_scale, bool accumulate, bool x_e5m2,
                       const void* swiglu_gu, bool tile_grid, bool clear_absmax, bool tiled) {
    if (x_e5m2 && (!fp8 || fuse_swiglu)) return hipErrorInvalidValue;
    if (tiled && !fp8 && (accumulate || swiglu_gu || q_absmax)) return hipErrorInvalidValue;
    const bool swi = swiglu_gu != nullptr;
    if (swi && (fuse_swiglu || accumulate)) return hipErrorInvalidValue;
    if (absmax && (fuse_swiglu || swi || N == 0) && clear_absmax) {
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
    a.ld_out = fuse_swiglu ? O / 2 : (swi ? 2 * O : O);
    a.aux = static_cast<const uint8_t*>(swiglu_gu);
    if (swi) a.absmax = absmax;
    a.tiles_m = fuse_swiglu ? (O / 2) / 128 : (O + kBM - 1) / kBM;
    a.tiles_n = (int)((N + kBN - 1) / kBN);
    a.q_absmax = q_absmax;
    a.q_scale = q_scale;
    const bool quant = fuse_swiglu && q_absmax;
    const int T = a.tiles_m * a.tiles_n;
    const int KT = a.K_bytes / kRowBytes;
    const dim3 grid((unsigned)(KT >= kAhead && !tile_grid ? persistent_grid(T) : T)), block(kThreads);
    const bool acc = accumulate && !fuse_swiglu;
    if (tiled && fp8) {
        if (swi && x_e5m2)
            hipLaunchKernelGGL((gemm_kernel<true, false, false, false, true, true, true>), grid, block, 0, s, a);
        else if (swi)
            hipLaunchKernelGGL((gemm_kernel<true, false, false, false, false, true, true>), grid, block, 0, s, a);
        else if (quant)
            hipLaunchKernelGGL((gemm_kernel<true, true, true, false, false, false, true>), grid, block, 0, s, a);
        else if (fuse_swiglu)
            hipLaunchKernelGGL((gemm_kernel<true, true, false, false, false, false, true>), grid, block, 0, s, a);
        else if (acc && x_e5m2)
            hipLaunchKernelGGL((gemm_kernel<true, false, false, true, true, false, true>), grid, block, 0, s, a);
        else if (acc)
            hipLaunchKernelGGL((gemm_kernel<true, false, false, true, false, false, true>), grid, block, 0, s, a);
        else if (x_e5m2)
            hipLaunchKernelGGL((gemm_kernel<true, false, false, false, true, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<true, false, false, false, false, false, true>), grid, block, 0, s, a);
    } else if (tiled) {
        if (fuse_swiglu)
            hipLaunchKernelGGL((gemm_kernel<false, true, false, false, false, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<false, false, false, false, false, false, true>), grid, block, 0, s, a);
    } else if (swi) {
        if (fp8 && x_e5m2) hipLaunchKernelGGL((gemm_kernel<true, false, false, false, true, true>), grid, block, 0, s, a);
        else if (fp8) hipLaunchKernelGGL((gemm_kernel<true, false, false, false, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<false, false, false, false, false, true>), grid, block, 0, s, a);
    } else if (fp8 && x_e5m2) {
        if (acc) hipLaunchKernelGGL((gemm_kernel<true, false, false, true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<true, false, false, false, true>), grid, block, 0, s, a);
    } else if (fp8) {
        if (quant) hipLaunchKernelGGL((gemm_kernel<true, true, true, false>), grid, block, 0, s, a);
        else if (fuse_swiglu) hipLaunchKernelGGL((gemm_kernel<true, true, false, false>), grid, block, 0, s, a);
        else if (acc) hipLaunchKernelGGL((gemm_kernel<true, false, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<true, false, false, false>), grid, block, 0, s, a);
    } else {
        if (quant) hipLaunchKernelGGL((gemm_kernel<false, true, true, false>), grid, block, 0, s, a);
        else if (fuse_swiglu) hipLaunchKernelGGL((gemm_kernel<false, true, false, false>), grid, block, 0, s, a);
        else if (acc) hipLaunchKernelGGL((gemm_kernel<false, false, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((gemm_kernel<false, false, false, false>), grid, block, 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse_swiglu || swi || !absmax) return e;
    return launch_absmax(absmax, static_cast<const uint16_t*>(out), N * (int64_t)O, s);
}

}  // namespace ffn
