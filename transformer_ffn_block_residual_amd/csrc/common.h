// Device helpers shared by the FFN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// The tiled operand layout of a K-contiguous GEMM operand [R, row_bytes]
// (row_bytes % 64 == 0): rows in groups of 64, each group one contiguous run
// of 64 row_bytes; inside a group, for each 64-byte K-step s and each 16-row
// sub-group i, the 1 KiB block at s * 4096 + i * 1024 holds exactly what one
// wave-wide 16-byte-per-lane load puts into the GEMM's LDS stage: lane l's 16
// bytes are chunk (l % 4) ^ (l / 16) of row 16 i + l / 4 at K-step s (the
// stage's XOR swizzle).  Byte offset of byte c of row r; an aligned 16-byte
// chunk of a row stays contiguous.
__device__ __forceinline__ int64_t tiled_offset(int64_t r, int64_t c, int64_t row_bytes) {
    const int rr = (int)(r & 63), lr = rr & 15;
    const int l = 4 * lr + ((int)((c >> 4) & 3) ^ (lr >> 2));
    return (r >> 6) * 64 * row_bytes + (c >> 6) * 4096 + (int64_t)((rr >> 4) * 1024 + l * 16) + (c & 15);
}

// bf16 bits (low 16 bits of u) -> fp32, exact.
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> two bf16 packed in one dword (a in the low half), round to nearest
// even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

// fp32 -> bf16 -> fp32: the value a bf16 store would hold.
__device__ __forceinline__ float round_bf16(float a) { return bf16lo(pack_bf16x2(a, 0.0f)); }

// SiLU(g) * u in fp32: g / (1 + exp(-g)) * u.  The exponential uses the
// hardware 2^x (v_exp_f32) and the division the hardware reciprocal; both are
// within a few fp32 ulps, far below the bf16 rounding that follows.
__device__ __forceinline__ float silu_mul(float g, float u) {
    float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Gradient of h = silu(g) * u at one element, dh given (every operand a bf16
// value held in fp32): s = 1 / (1 + exp(-g)),
//   dg = dh * u * s * (1 + g * (1 - s)),  du = dh * g * s   (fp32, unrounded)
// One function for the SwiGLU backward pass and the epilogue that fuses it
// into the data-gradient GEMM, so both round the same fp32 values.
__device__ __forceinline__ void swiglu_bwd_pair(float d, float g, float u, float& dg, float& du) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    const float sg = __builtin_amdgcn_rcpf(1.0f + e);
    dg = d * u * sg * (1.0f + g * (1.0f - sg));
    du = d * g * sg;
}

// x clamped to [-m, m]; a NaN stays NaN (fmaxf/fminf alone would turn it into
// -m, a finite code).
__device__ __forceinline__ float clamp_keep_nan(float x, float m) {
    return x != x ? x : __builtin_fminf(__builtin_fmaxf(x, -m), m);
}

// Four fp32 -> four e4m3 codes in one dword (a in the lowest byte).  Values are
// clamped to +-448 first so the conversion never depends on an overflow mode;
// v_cvt_pk_fp8_f32 rounds to nearest even and turns a NaN into a NaN code.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    a = clamp_keep_nan(a, kE4M3Max);
    b = clamp_keep_nan(b, kE4M3Max);
    c = clamp_keep_nan(c, kE4M3Max);
    d = clamp_keep_nan(d, kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Four fp32 -> four e5m2 codes in one dword (a in the lowest byte), clamped
// to +-57344 first (NaN kept); v_cvt_pk_bf8_f32 rounds to nearest even.
__device__ __forceinline__ uint32_t pack_e5m2x4(float a, float b, float c, float d) {
    a = clamp_keep_nan(a, kE5M2Max);
    b = clamp_keep_nan(b, kE5M2Max);
    c = clamp_keep_nan(c, kE5M2Max);
    d = clamp_keep_nan(d, kE5M2Max);
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Per-tensor FP8 scale pair from an abs-max: the dequantisation factor
// absmax/max and its quantisation inverse max/absmax (max = 448 for e4m3,
// 57344 for e5m2), both IEEE fp32 quotients; 1 and 1 for an all-zero tensor.
// A NaN abs-max gives NaN for both, so every code of the tensor is NaN.
__device__ __forceinline__ void scale_pair(float am, float& scale, float& inv, float fmax = kE4M3Max) {
    if (am == 0.0f) {
        scale = 1.0f;
        inv = 1.0f;
    } else {
        scale = am / fmax;
        inv = fmax / am;
    }
}

// Bytes 0,1 (hi=false) or 2,3 (hi=true) of a dword of e4m3 codes -> fp32, exact.
__device__ __forceinline__ f32x2_t e4m3x2_to_f32(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// Bytes 0,1 (hi=false) or 2,3 (hi=true) of a dword of e4m3 codes -> a packed
// bf16 pair (element 0 in the low half), exact.
__device__ __forceinline__ bf16x2_t e4m3x2_to_bf16(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

// c + w.lo * x.lo + w.hi * x.hi on packed bf16 pairs, fp32 accumulation
// (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), c,
                                           false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Abs-max accumulation: m = max(m, |v|) as the unsigned order of the bit
// patterns of non-negative floats.  For numbers this is the IEEE order; a NaN
// pattern lies above +inf, so a NaN anywhere in a tensor makes its abs-max NaN
// (fmaxf would skip it).  m must be non-negative or NaN.
__device__ __forceinline__ float absmax_acc(float m, float v) {
    return __uint_as_float(max(__float_as_uint(m), __float_as_uint(v) & 0x7fffffffu));
}

// The same maximum over the 64 lanes (every value non-negative or NaN).
__device__ __forceinline__ float wave_absmax(float v) {
    unsigned int u = __float_as_uint(v);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) u = max(u, (unsigned int)__shfl_xor((int)u, m, kWave));
    return __uint_as_float(u);
}

// max into a non-negative fp32 in global memory: for v >= 0 the IEEE order is
// the unsigned order of the bit patterns (a NaN pattern above all of them), so
// an integer atomic max is exact and independent of the order in which blocks
// arrive.  The stored maximum only
// grows while blocks commit, so the atomic is skipped when the value already
// there (read from L2, device scope) is at least v: a stale read can only
// cost an unneeded atomic, never skip a needed one.  Thousands of blocks that
// finish together otherwise queue on the one address.
__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
    unsigned int* u = reinterpret_cast<unsigned int*>(p);
    const unsigned int cur = __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(v) > cur) atomicMax(u, __float_as_uint(v));
}

// Block-wide abs-max of a per-thread value (non-negative or NaN, the order of
// absmax_acc), then one atomic per block.  All threads of the block must call
// it.  `red` is LDS scratch of at least nwaves floats.
__device__ __forceinline__ void block_absmax_commit(float v, float* red, float* out) {
    v = wave_absmax(v);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    if (lane == 0) red[wid] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
        for (int i = 1; i < (int)(blockDim.x / kWave); ++i) m = absmax_acc(m, red[i]);
        atomic_max_nonneg(out, m);
    }
}

}  // namespace ffn
