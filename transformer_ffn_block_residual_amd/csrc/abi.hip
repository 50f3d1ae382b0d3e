// C ABI of libffn.so (declared in include/ffn.h): argument validation, then the
// kernel launches.  Validation touches no HIP API, so every error path can be
// exercised on a machine without a GPU.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "../../include/ffn.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

ffn_status_t fail(ffn_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

ffn_status_t hip_status(hipError_t e, const char* fn) {
    if (e == hipSuccess) return FFN_OK;
    return fail(FFN_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

#define REQUIRE(ptr)                                                                  \
    do {                                                                              \
        if (!(ptr)) return fail(FFN_ERR_INVALID, "%s: %s is NULL", __func__, #ptr);   \
    } while (0)
#define ALIGNED(ptr)                                                                                   \
    do {                                                                                               \
        if ((ptr) && misaligned(ptr))                                                                  \
            return fail(FFN_ERR_UNSUPPORTED, "%s: %s is not 16-byte aligned", __func__, #ptr);         \
    } while (0)
#define NONNEG(v)                                                                                      \
    do {                                                                                               \
        if ((v) < 0) return fail(FFN_ERR_INVALID, "%s: %s = %lld is negative", __func__, #v, (long long)(v)); \
    } while (0)

const int64_t kMaxDim = 1 << 20;

// The workspace of ffn_decode_gemv_packed_noalloc: a fixed array in device
// memory that every call on a device shares (each device holds its own copy
// from the library's load until the process ends).  In host code the name
// `scratch` is only a stand-in for the symbol: kernels are given its device
// address, looked up once per device with hipGetSymbolAddress.
constexpr int64_t kNoAllocScratchBytes = (int64_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call on that device; threads that race here store the same address).
hipError_t scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* ffn_last_error(void) { return g_err; }

const char* ffn_version(void) { return "ffn-mi355x 0.1 (gfx950)"; }

static int64_t tiled_bytes(int64_t rows, int64_t row_bytes) { return (rows + 63) / 64 * 64 * row_bytes; }

static bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    const uint8_t *pa = static_cast<const uint8_t*>(a), *pb = static_cast<const uint8_t*>(b);
    return a && b && na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

static ffn_status_t rmsnorm_entry(const char* fn, void* y, float* rstd, void* residual_out, float* absmax,
                                  const void* inp, const void* addend, const void* weight, float eps, int64_t N,
                                  int64_t C, hipStream_t stream, bool clear_absmax, bool tiled_y = false) {
    if (!y) return fail(FFN_ERR_INVALID, "%s: y is NULL", fn);
    if (!rstd) return fail(FFN_ERR_INVALID, "%s: rstd is NULL", fn);
    if (!inp) return fail(FFN_ERR_INVALID, "%s: inp is NULL", fn);
    if (!weight) return fail(FFN_ERR_INVALID, "%s: weight is NULL", fn);
    if (N < 0 || C < 0) return fail(FFN_ERR_INVALID, "%s: negative size", fn);
    if (addend && !residual_out) return fail(FFN_ERR_INVALID, "%s: addend given without residual_out", fn);
    if (!addend && residual_out) return fail(FFN_ERR_INVALID, "%s: residual_out given without addend", fn);
    if (!(eps >= 0.0f)) return fail(FFN_ERR_INVALID, "%s: eps must be >= 0", fn);
    if (C < 8 || C > 16384 || C % 8 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "%s: C = %lld (need 8 <= C <= 16384, C %% 8 == 0)", fn, (long long)C);
    if (N > (int64_t)1 << 31) return fail(FFN_ERR_UNSUPPORTED, "%s: N too large", fn);
    if (misaligned(y) || misaligned(inp) || misaligned(addend) || misaligned(residual_out) || misaligned(weight))
        return fail(FFN_ERR_UNSUPPORTED, "%s: a buffer is not 16-byte aligned", fn);
    if (residual_out && (residual_out == y || residual_out == addend))
        return fail(FFN_ERR_INVALID, "%s: residual_out may alias only inp", fn);
    if (tiled_y) {
        // a row's tiled chunks land among the bytes of its whole 64-row group
        if (C % 32 != 0) return fail(FFN_ERR_UNSUPPORTED, "%s: C = %lld (need C %% 32 == 0)", fn, (long long)C);
        const int64_t ny = tiled_bytes(N, 2 * C), nx = N * C * 2;
        if (overlaps(y, ny, inp, nx) || overlaps(y, ny, addend, nx) || overlaps(y, ny, residual_out, nx))
            return fail(FFN_ERR_INVALID, "%s: the tiled y must not overlap inp, addend or residual_out", fn);
    }
    return hip_status(ffn::launch_rmsnorm((uint16_t*)y, rstd, (uint16_t*)residual_out, absmax,
                                          (const uint16_t*)inp, (const uint16_t*)addend, (const uint16_t*)weight,
                                          eps, N, (int)C, stream, clear_absmax, tiled_y),
                      fn);
}

ffn_status_t ffn_rmsnorm_fwd(void* y, float* rstd, void* residual_out, float* absmax, const void* inp,
                             const void* addend, const void* weight, float eps, int64_t N, int64_t C,
                             hipStream_t stream) {
    return rmsnorm_entry("ffn_rmsnorm_fwd", y, rstd, residual_out, absmax, inp, addend, weight, eps, N, C, stream,
                         true);
}

ffn_status_t ffn_rmsnorm_fwd_tiled(void* y, float* rstd, void* residual_out, float* absmax, const void* inp,
                                   const void* addend, const void* weight, float eps, int64_t N, int64_t C,
                                   hipStream_t stream) {
    return rmsnorm_entry("ffn_rmsnorm_fwd_tiled", y, rstd, residual_out, absmax, inp, addend, weight, eps, N, C,
                         stream, true, true);
}

ffn_status_t ffn_rmsnorm_fwd_acc(void* y, float* rstd, void* residual_out, float* absmax, const void* inp,
                                 const void* addend, const void* weight, float eps, int64_t N, int64_t C,
                                 hipStream_t stream) {
    REQUIRE(absmax);
    return rmsnorm_entry("ffn_rmsnorm_fwd_acc", y, rstd, residual_out, absmax, inp, addend, weight, eps, N, C,
                         stream, false);
}

ffn_status_t ffn_quant_absmax(uint8_t* q, float* scale, float* absmax, const void* x, int64_t n,
                              int compute_absmax, hipStream_t stream) {
    REQUIRE(q);
    REQUIRE(scale);
    REQUIRE(absmax);
    REQUIRE(x);
    NONNEG(n);
    if ((void*)scale == (void*)absmax) return fail(FFN_ERR_INVALID, "ffn_quant_absmax: scale and absmax alias");
    if (n > ((int64_t)1 << 36)) return fail(FFN_ERR_UNSUPPORTED, "ffn_quant_absmax: n too large");
    ALIGNED(q);
    ALIGNED(x);
    return hip_status(ffn::launch_quant(q, scale, absmax, (const uint16_t*)x, n, compute_absmax != 0, stream),
                      "ffn_quant_absmax");
}

ffn_status_t ffn_quant_absmax_clear(uint8_t* q, float* scale, const float* absmax, const void* x, int64_t n,
                                    float* clear, hipStream_t stream) {
    REQUIRE(q);
    REQUIRE(scale);
    REQUIRE(absmax);
    REQUIRE(x);
    REQUIRE(clear);
    NONNEG(n);
    if ((const float*)scale == absmax || (const float*)clear == absmax || clear == scale)
        return fail(FFN_ERR_INVALID, "ffn_quant_absmax_clear: scale, absmax and clear must be three words");
    if (n > ((int64_t)1 << 36)) return fail(FFN_ERR_UNSUPPORTED, "ffn_quant_absmax_clear: n too large");
    ALIGNED(q);
    ALIGNED(x);
    return hip_status(ffn::launch_quant(q, scale, const_cast<float*>(absmax), (const uint16_t*)x, n, false, stream,
                                        clear),
                      "ffn_quant_absmax_clear");
}

ffn_status_t ffn_quant_rows(uint8_t* q, float* row_scale, const void* w, int64_t rows, int64_t cols,
                            hipStream_t stream) {
    REQUIRE(q);
    REQUIRE(row_scale);
    REQUIRE(w);
    NONNEG(rows);
    NONNEG(cols);
    if (cols < 8 || cols % 8 != 0 || cols > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_quant_rows: cols = %lld (need cols %% 8 == 0)", (long long)cols);
    if (rows > (int64_t)1 << 31) return fail(FFN_ERR_UNSUPPORTED, "ffn_quant_rows: rows too large");
    ALIGNED(q);
    ALIGNED(w);
    return hip_status(ffn::launch_quant_rows(q, row_scale, (const uint16_t*)w, rows, (int)cols, stream),
                      "ffn_quant_rows");
}

static ffn_status_t check_gemm_dims(const char* fn, int64_t N, int64_t K, int64_t O, int elt) {
    if (K < 128 || K % 128 != 0 || K > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "%s: reduction size %lld must be a positive multiple of 128", fn,
                    (long long)K);
    if (O < 128 || O % 128 != 0 || O > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "%s: output features %lld must be a positive multiple of 128", fn,
                    (long long)O);
    // byte offsets inside one operand are kept in 32 bits
    if (O * K * elt >= ((int64_t)1 << 32) || N * K * elt >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "%s: an operand exceeds 4 GiB", fn);
    if (N > ((int64_t)1 << 31) - 256) return fail(FFN_ERR_UNSUPPORTED, "%s: N too large", fn);
    return FFN_OK;
}

ffn_status_t ffn_gateup(void* out, float* out_absmax, const void* x, const float* x_scale, const void* w,
                        const float* w_scale, ffn_dtype_t dtype, int fuse_swiglu, int64_t N, int64_t C, int64_t H,
                        hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(x);
    REQUIRE(w);
    NONNEG(N);
    NONNEG(C);
    NONNEG(H);
    if (dtype != FFN_BF16 && dtype != FFN_E4M3) return fail(FFN_ERR_INVALID, "ffn_gateup: unknown dtype %d", (int)dtype);
    if (dtype == FFN_E4M3) {
        REQUIRE(x_scale);
        REQUIRE(w_scale);
    }
    // the abs-max is cleared before the scales are read: they must be other words
    if (out_absmax && (out_absmax == x_scale || out_absmax == w_scale))
        return fail(FFN_ERR_INVALID, "ffn_gateup: out_absmax must not alias x_scale or w_scale");
    const int elt = dtype == FFN_E4M3 ? 1 : 2;
    if (ffn_status_t st = check_gemm_dims("ffn_gateup", N, C, 2 * H, elt)) return st;
    if (H % 128 != 0) return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup: H = %lld must be a multiple of 128", (long long)H);
    ALIGNED(out);
    ALIGNED(x);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(out, out_absmax, x, x_scale, w, w_scale, dtype == FFN_E4M3, fuse_swiglu != 0,
                                       N, (int)C, (int)(2 * H), stream),
                      "ffn_gateup");
}

ffn_status_t ffn_gateup_acc(void* h, float* h_absmax, const void* x, const float* x_scale, const void* w,
                            const float* w_scale, ffn_dtype_t dtype, int64_t N, int64_t C, int64_t H,
                            hipStream_t stream) {
    REQUIRE(h);
    REQUIRE(h_absmax);
    REQUIRE(x);
    REQUIRE(w);
    NONNEG(N);
    NONNEG(C);
    NONNEG(H);
    if (dtype != FFN_BF16 && dtype != FFN_E4M3)
        return fail(FFN_ERR_INVALID, "ffn_gateup_acc: unknown dtype %d", (int)dtype);
    if (dtype == FFN_E4M3) {
        REQUIRE(x_scale);
        REQUIRE(w_scale);
    }
    if (h_absmax == x_scale || h_absmax == w_scale)
        return fail(FFN_ERR_INVALID, "ffn_gateup_acc: h_absmax must not alias x_scale or w_scale");
    const int elt = dtype == FFN_E4M3 ? 1 : 2;
    if (ffn_status_t st = check_gemm_dims("ffn_gateup_acc", N, C, 2 * H, elt)) return st;
    if (H % 128 != 0) return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup_acc: H = %lld must be a multiple of 128", (long long)H);
    ALIGNED(h);
    ALIGNED(x);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(h, h_absmax, x, x_scale, w, w_scale, dtype == FFN_E4M3, true, N, (int)C,
                                       (int)(2 * H), stream, nullptr, nullptr, false, false, nullptr, false, false),
                      "ffn_gateup_acc");
}

ffn_status_t ffn_gateup_swiglu_quant(uint8_t* q, float* q_scale, float* h_absmax, const float* h_absmax_known,
                                     const void* x, const float* x_scale, const void* w, const float* w_scale,
                                     ffn_dtype_t dtype, int64_t N, int64_t C, int64_t H, hipStream_t stream) {
    REQUIRE(q);
    REQUIRE(q_scale);
    REQUIRE(h_absmax_known);
    REQUIRE(x);
    REQUIRE(w);
    NONNEG(N);
    NONNEG(C);
    NONNEG(H);
    if (dtype != FFN_BF16 && dtype != FFN_E4M3)
        return fail(FFN_ERR_INVALID, "ffn_gateup_swiglu_quant: unknown dtype %d", (int)dtype);
    if (dtype == FFN_E4M3) {
        REQUIRE(x_scale);
        REQUIRE(w_scale);
    }
    if (h_absmax_known == h_absmax || h_absmax_known == q_scale)
        return fail(FFN_ERR_INVALID, "ffn_gateup_swiglu_quant: h_absmax_known must not alias h_absmax or q_scale");
    if ((h_absmax && (h_absmax == x_scale || h_absmax == w_scale)) || q_scale == x_scale || q_scale == w_scale)
        return fail(FFN_ERR_INVALID, "ffn_gateup_swiglu_quant: h_absmax and q_scale must not alias x_scale or w_scale");
    const int elt = dtype == FFN_E4M3 ? 1 : 2;
    if (ffn_status_t st = check_gemm_dims("ffn_gateup_swiglu_quant", N, C, 2 * H, elt)) return st;
    if (H % 128 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup_swiglu_quant: H = %lld must be a multiple of 128", (long long)H);
    ALIGNED(q);
    ALIGNED(x);
    ALIGNED(w);
    if (N == 0) {
        // no rows: the abs-max of no elements is 0, and the scale is still
        // published from the known abs-max (the quantisation kernel's n = 0 path)
        if (h_absmax) {
            const ffn_status_t st = hip_status(ffn::launch_fill(h_absmax, 1, 0.0f, stream), "ffn_gateup_swiglu_quant");
            if (st != FFN_OK) return st;
        }
        return hip_status(ffn::launch_quant(nullptr, q_scale, const_cast<float*>(h_absmax_known), nullptr, 0, false,
                                            stream),
                          "ffn_gateup_swiglu_quant");
    }
    return hip_status(ffn::launch_gemm(q, h_absmax, x, x_scale, w, w_scale, dtype == FFN_E4M3, true, N, (int)C,
                                       (int)(2 * H), stream, h_absmax_known, q_scale),
                      "ffn_gateup_swiglu_quant");
}

ffn_status_t ffn_swiglu(void* h, float* absmax, const void* gateup, int64_t N, int64_t H, hipStream_t stream) {
    REQUIRE(h);
    REQUIRE(gateup);
    NONNEG(N);
    NONNEG(H);
    if (H < 8 || H % 8 != 0 || H > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_swiglu: H = %lld (need H %% 8 == 0)", (long long)H);
    if (N * H > ((int64_t)1 << 36)) return fail(FFN_ERR_UNSUPPORTED, "ffn_swiglu: tensor too large");
    ALIGNED(h);
    ALIGNED(gateup);
    return hip_status(ffn::launch_swiglu((uint16_t*)h, absmax, (const uint16_t*)gateup, N, (int)H, stream),
                      "ffn_swiglu");
}

ffn_status_t ffn_down(void* out, const void* h, const float* h_scale, const void* w, const float* w_scale,
                      ffn_dtype_t dtype, int64_t N, int64_t H, int64_t C, hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(h);
    REQUIRE(w);
    NONNEG(N);
    NONNEG(H);
    NONNEG(C);
    if (dtype != FFN_BF16 && dtype != FFN_E4M3) return fail(FFN_ERR_INVALID, "ffn_down: unknown dtype %d", (int)dtype);
    if (dtype == FFN_E4M3) {
        REQUIRE(h_scale);
        REQUIRE(w_scale);
    }
    const int elt = dtype == FFN_E4M3 ? 1 : 2;
    if (ffn_status_t st = check_gemm_dims("ffn_down", N, H, C, elt)) return st;
    ALIGNED(out);
    ALIGNED(h);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(out, nullptr, h, h_scale, w, w_scale, dtype == FFN_E4M3, false, N, (int)H,
                                       (int)C, stream),
                      "ffn_down");
}

// ---- tiled operands (whole 64-row groups; common.h, tiled_offset)

int64_t ffn_tile_bytes(int64_t rows, int64_t row_bytes) {
    if (rows < 0 || row_bytes < 0 || row_bytes % 64 != 0 || row_bytes > ((int64_t)1 << 21) ||
        rows > ((int64_t)1 << 40))
        return -1;
    return tiled_bytes(rows, row_bytes);
}

ffn_status_t ffn_tile_pack(void* out, const void* in, int64_t rows, int64_t row_bytes, hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(in);
    NONNEG(rows);
    NONNEG(row_bytes);
    if (row_bytes < 64 || row_bytes % 64 != 0 || row_bytes > ((int64_t)1 << 21))
        return fail(FFN_ERR_UNSUPPORTED, "ffn_tile_pack: row_bytes = %lld (need a multiple of 64, 64 .. 2^21)",
                    (long long)row_bytes);
    if (rows > ((int64_t)1 << 36) / row_bytes || tiled_bytes(rows, row_bytes) >= ((int64_t)1 << 36))
        return fail(FFN_ERR_UNSUPPORTED, "ffn_tile_pack: operand too large");
    ALIGNED(out);
    ALIGNED(in);
    const uint8_t* i8 = static_cast<const uint8_t*>(in);
    const uint8_t* o8 = static_cast<const uint8_t*>(out);
    if (o8 < i8 + rows * row_bytes && i8 < o8 + tiled_bytes(rows, row_bytes))
        return fail(FFN_ERR_INVALID, "ffn_tile_pack: out overlaps in");
    return hip_status(ffn::launch_tile_pack(static_cast<uint8_t*>(out), i8, rows, row_bytes, stream),
                      "ffn_tile_pack");
}

ffn_status_t ffn_quant_absmax_clear_tiled(uint8_t* q, float* scale, const float* absmax, const void* x,
                                          int64_t rows, int64_t cols, float* clear, hipStream_t stream) {
    REQUIRE(q);
    REQUIRE(scale);
    REQUIRE(absmax);
    REQUIRE(x);
    NONNEG(rows);
    NONNEG(cols);
    if ((const float*)scale == absmax || (clear && ((const float*)clear == absmax || clear == scale)))
        return fail(FFN_ERR_INVALID, "ffn_quant_absmax_clear_tiled: scale, absmax and clear must be distinct words");
    if (cols < 128 || cols % 128 != 0 || cols > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_quant_absmax_clear_tiled: cols = %lld (need a positive multiple of 128)",
                    (long long)cols);
    // the quantiser's thread index (64 per row pair and 8 K-steps) stays in 32 bits
    if (rows > ((int64_t)1 << 36) / cols || tiled_bytes(rows, cols) > ((int64_t)1 << 36) ||
        (rows + 1) / 2 * ((cols / 64 + 7) / 8) * 64 >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "ffn_quant_absmax_clear_tiled: too large");
    // a row's tiled codes land among the bytes of its whole 64-row group
    if (overlaps(q, tiled_bytes(rows, cols), x, rows * cols * 2))
        return fail(FFN_ERR_INVALID, "ffn_quant_absmax_clear_tiled: q must not overlap x");
    ALIGNED(q);
    ALIGNED(x);
    return hip_status(ffn::launch_quant_tiled(q, scale, const_cast<float*>(absmax), (const uint16_t*)x, rows, cols,
                                              stream, clear),
                      "ffn_quant_absmax_clear_tiled");
}

// The checks of the row-major entry point, plus the tiled token operand's
// whole groups within the 32-bit offsets of one operand.
static ffn_status_t check_tiled_gemm(const char* fn, int64_t N, int64_t K, int64_t O, int elt = 1) {
    if (ffn_status_t st = check_gemm_dims(fn, N, K, O, elt)) return st;
    if (tiled_bytes(N, K * elt) >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "%s: an operand exceeds 4 GiB", fn);
    return FFN_OK;
}

ffn_status_t ffn_gateup_acc_tiled(void* h, float* h_absmax, const uint8_t* x, const float* x_scale, const uint8_t* w,
                                  const float* w_scale, int64_t N, int64_t C, int64_t H, hipStream_t stream) {
    REQUIRE(h);
    REQUIRE(h_absmax);
    REQUIRE(x);
    REQUIRE(x_scale);
    REQUIRE(w);
    REQUIRE(w_scale);
    NONNEG(N);
    NONNEG(C);
    NONNEG(H);
    if (h_absmax == x_scale || h_absmax == w_scale)
        return fail(FFN_ERR_INVALID, "ffn_gateup_acc_tiled: h_absmax must not alias x_scale or w_scale");
    if (ffn_status_t st = check_tiled_gemm("ffn_gateup_acc_tiled", N, C, 2 * H)) return st;
    if (H % 128 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup_acc_tiled: H = %lld must be a multiple of 128", (long long)H);
    ALIGNED(h);
    ALIGNED(x);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(h, h_absmax, x, x_scale, w, w_scale, true, true, N, (int)C, (int)(2 * H),
                                       stream, nullptr, nullptr, false, false, nullptr, false, false, true),
                      "ffn_gateup_acc_tiled");
}

ffn_status_t ffn_gateup_swiglu_quant_tiled(uint8_t* q, float* q_scale, float* h_absmax, const float* h_absmax_known,
                                           const uint8_t* x, const float* x_scale, const uint8_t* w,
                                           const float* w_scale, int64_t N, int64_t C, int64_t H,
                                           hipStream_t stream) {
    REQUIRE(q);
    REQUIRE(q_scale);
    REQUIRE(h_absmax_known);
    REQUIRE(x);
    REQUIRE(x_scale);
    REQUIRE(w);
    REQUIRE(w_scale);
    NONNEG(N);
    NONNEG(C);
    NONNEG(H);
    if (h_absmax_known == h_absmax || h_absmax_known == q_scale)
        return fail(FFN_ERR_INVALID,
                    "ffn_gateup_swiglu_quant_tiled: h_absmax_known must not alias h_absmax or q_scale");
    if ((h_absmax && (h_absmax == x_scale || h_absmax == w_scale)) || q_scale == x_scale || q_scale == w_scale)
        return fail(FFN_ERR_INVALID,
                    "ffn_gateup_swiglu_quant_tiled: h_absmax and q_scale must not alias x_scale or w_scale");
    if (ffn_status_t st = check_tiled_gemm("ffn_gateup_swiglu_quant_tiled", N, C, 2 * H)) return st;
    if (H % 128 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup_swiglu_quant_tiled: H = %lld must be a multiple of 128",
                    (long long)H);
    if (tiled_bytes(N, H) >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup_swiglu_quant_tiled: the codes of h exceed 4 GiB");
    ALIGNED(q);
    ALIGNED(x);
    ALIGNED(w);
    if (N == 0) {
        // as ffn_gateup_swiglu_quant: abs-max 0, the scale from the known abs-max
        if (h_absmax) {
            const ffn_status_t st =
                hip_status(ffn::launch_fill(h_absmax, 1, 0.0f, stream), "ffn_gateup_swiglu_quant_tiled");
            if (st != FFN_OK) return st;
        }
        return hip_status(ffn::launch_quant(nullptr, q_scale, const_cast<float*>(h_absmax_known), nullptr, 0, false,
                                            stream),
                          "ffn_gateup_swiglu_quant_tiled");
    }
    return hip_status(ffn::launch_gemm(q, h_absmax, x, x_scale, w, w_scale, true, true, N, (int)C, (int)(2 * H),
                                       stream, h_absmax_known, q_scale, false, false, nullptr, false, true, true),
                      "ffn_gateup_swiglu_quant_tiled");
}

ffn_status_t ffn_down_tiled(void* out, const uint8_t* h, const float* h_scale, const uint8_t* w,
                            const float* w_scale, int64_t N, int64_t H, int64_t C, hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(h);
    REQUIRE(h_scale);
    REQUIRE(w);
    REQUIRE(w_scale);
    NONNEG(N);
    NONNEG(H);
    NONNEG(C);
    if (ffn_status_t st = check_tiled_gemm("ffn_down_tiled", N, H, C)) return st;
    ALIGNED(out);
    ALIGNED(h);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(out, nullptr, h, h_scale, w, w_scale, true, false, N, (int)H, (int)C, stream,
                                       nullptr, nullptr, false, false, nullptr, false, true, true),
                      "ffn_down_tiled");
}

ffn_status_t ffn_gateup_tiled_bf16(void* h, float* h_absmax, const void* x, const void* w, int64_t N, int64_t C,
                                   int64_t H, hipStream_t stream) {
    REQUIRE(h);
    REQUIRE(x);
    REQUIRE(w);
    NONNEG(N);
    NONNEG(C);
    NONNEG(H);
    if (ffn_status_t st = check_tiled_gemm("ffn_gateup_tiled_bf16", N, C, 2 * H, 2)) return st;
    if (H % 128 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_gateup_tiled_bf16: H = %lld must be a multiple of 128", (long long)H);
    ALIGNED(h);
    ALIGNED(x);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(h, h_absmax, x, nullptr, w, nullptr, false, true, N, (int)C, (int)(2 * H),
                                       stream, nullptr, nullptr, false, false, nullptr, false, true, true),
                      "ffn_gateup_tiled_bf16");
}

ffn_status_t ffn_down_tiled_bf16(void* out, const void* h, const void* w, int64_t N, int64_t H, int64_t C,
                                 hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(h);
    REQUIRE(w);
    NONNEG(N);
    NONNEG(H);
    NONNEG(C);
    if (ffn_status_t st = check_tiled_gemm("ffn_down_tiled_bf16", N, H, C, 2)) return st;
    ALIGNED(out);
    ALIGNED(h);
    ALIGNED(w);
    return hip_status(ffn::launch_gemm(out, nullptr, h, nullptr, w, nullptr, false, false, N, (int)H, (int)C, stream,
                                       nullptr, nullptr, false, false, nullptr, false, true, true),
                      "ffn_down_tiled_bf16");
}

// Checks shared by the decode entry points (elt: weight bytes per element).
static ffn_status_t check_decode(const char* fn, const void* out, const void* h, const void* x, const void* wg,
                                 const void* wu, const void* wd, int64_t M, int64_t C, int64_t H, int elt,
                                 int64_t max_m) {
    if (!out || !h || !x || !wg || !wu || !wd) return fail(FFN_ERR_INVALID, "%s: a required pointer is NULL", fn);
    if (M < 0 || C < 0 || H < 0) return fail(FFN_ERR_INVALID, "%s: negative size", fn);
    if (M > max_m) return fail(FFN_ERR_UNSUPPORTED, "%s: M = %lld > %lld", fn, (long long)M, (long long)max_m);
    if (C < 128 || C % 128 != 0 || C > kMaxDim || H < 128 || H % 128 != 0 || H > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "%s: C = %lld, H = %lld must be positive multiples of 128", fn,
                    (long long)C, (long long)H);
    if (C * H * elt >= ((int64_t)1 << 31)) return fail(FFN_ERR_UNSUPPORTED, "%s: weights exceed 2 GiB", fn);
    if (misaligned(out) || misaligned(h) || misaligned(x) || misaligned(wg) || misaligned(wu) || misaligned(wd))
        return fail(FFN_ERR_UNSUPPORTED, "%s: a buffer is not 16-byte aligned", fn);
    if (h == x || out == h) return fail(FFN_ERR_INVALID, "%s: h must not alias x or out", fn);
    return FFN_OK;
}

ffn_status_t ffn_decode_gemv(void* out, void* h, const void* x, const uint8_t* w_gate, const float* s_gate,
                             const uint8_t* w_up, const float* s_up, const uint8_t* w_down, const float* s_down,
                             int64_t M, int64_t C, int64_t H, hipStream_t stream) {
    REQUIRE(s_gate);
    REQUIRE(s_up);
    REQUIRE(s_down);
    if (ffn_status_t st = check_decode("ffn_decode_gemv", out, h, x, w_gate, w_up, w_down, M, C, H, 1, 32)) return st;
    return hip_status(ffn::launch_decode((uint16_t*)out, (uint16_t*)h, nullptr, (const uint16_t*)x, w_gate, s_gate,
                                         w_up, s_up, w_down, s_down, ffn::kDecodeSplitSilu, false, (int)M, (int)C,
                                         (int)H, stream),
                      "ffn_decode_gemv");
}

ffn_status_t ffn_decode_gemv_arm(void* out, void* h, void* gu, const void* x, const uint8_t* w_gate,
                                 const float* s_gate, const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                                 const float* s_down, ffn_decode_arm_t arm, int64_t M, int64_t C, int64_t H,
                                 hipStream_t stream) {
    REQUIRE(s_gate);
    REQUIRE(s_up);
    REQUIRE(s_down);
    if (arm != FFN_DECODE_SPLIT_SILU && arm != FFN_DECODE_SILU_INPUT && arm != FFN_DECODE_PER_PROJECTION)
        return fail(FFN_ERR_INVALID, "ffn_decode_gemv_arm: unknown arm %d", (int)arm);
    const int64_t max_m = arm == FFN_DECODE_SPLIT_SILU ? 32 : 4;
    if (ffn_status_t st = check_decode("ffn_decode_gemv_arm", out, h, x, w_gate, w_up, w_down, M, C, H, 1, max_m))
        return st;
    if (arm != FFN_DECODE_SPLIT_SILU) {
        REQUIRE(gu);
        ALIGNED(gu);
        if (gu == x || gu == out || gu == h)
            return fail(FFN_ERR_INVALID, "ffn_decode_gemv_arm: gu must not alias x, out or h");
    }
    return hip_status(ffn::launch_decode((uint16_t*)out, (uint16_t*)h, (uint16_t*)gu, (const uint16_t*)x, w_gate,
                                         s_gate, w_up, s_up, w_down, s_down, (int)arm, false, (int)M, (int)C, (int)H,
                                         stream),
                      "ffn_decode_gemv_arm");
}

ffn_status_t ffn_decode_gemv_bf16(void* out, void* h, const void* x, const void* w_gate, const void* w_up,
                                  const void* w_down, int64_t M, int64_t C, int64_t H, hipStream_t stream) {
    if (ffn_status_t st = check_decode("ffn_decode_gemv_bf16", out, h, x, w_gate, w_up, w_down, M, C, H, 2, 4))
        return st;
    return hip_status(ffn::launch_decode((uint16_t*)out, (uint16_t*)h, nullptr, (const uint16_t*)x,
                                         (const uint8_t*)w_gate, nullptr, (const uint8_t*)w_up, nullptr,
                                         (const uint8_t*)w_down, nullptr, ffn::kDecodeSplitSilu, true, (int)M, (int)C,
                                         (int)H, stream),
                      "ffn_decode_gemv_bf16");
}

ffn_status_t ffn_decode_pack_weight(uint8_t* packed, const uint8_t* w, int64_t rows, int64_t cols,
                                    hipStream_t stream) {
    REQUIRE(packed);
    REQUIRE(w);
    if (rows < 0 || cols < 0) return fail(FFN_ERR_INVALID, "ffn_decode_pack_weight: negative size");
    if (rows % 16 != 0 || cols % 128 != 0 || cols > kMaxDim || rows > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "ffn_decode_pack_weight: rows = %lld must be a multiple of 16 and cols = "
                    "%lld of 128", (long long)rows, (long long)cols);
    if (misaligned(packed) || misaligned(w))
        return fail(FFN_ERR_UNSUPPORTED, "ffn_decode_pack_weight: a buffer is not 16-byte aligned");
    if ((const void*)packed == (const void*)w)
        return fail(FFN_ERR_INVALID, "ffn_decode_pack_weight: packed must not alias w");
    return hip_status(ffn::launch_pack_weight(packed, w, rows, (int)cols, stream), "ffn_decode_pack_weight");
}

int64_t ffn_decode_packed_workspace_bytes(int64_t M, int64_t C, int64_t H) {
    if (M < 0 || M > 32 || C < 0 || H < 0 || C > kMaxDim || H > kMaxDim) return -1;
    return ffn::decode_packed_ws_elems((int)M, (int)C, (int)H) * 2;
}

ffn_status_t ffn_decode_gemv_packed(void* out, void* h, void* workspace, const void* x, const uint8_t* w_gate,
                                    const float* s_gate, const uint8_t* w_up, const float* s_up,
                                    const uint8_t* w_down, const float* s_down, int64_t M, int64_t C, int64_t H,
                                    hipStream_t stream) {
    REQUIRE(s_gate);
    REQUIRE(s_up);
    REQUIRE(s_down);
    REQUIRE(workspace);
    if (ffn_status_t st = check_decode("ffn_decode_gemv_packed", out, h, x, w_gate, w_up, w_down, M, C, H, 1, 32))
        return st;
    ALIGNED(workspace);
    if (workspace == out || workspace == h || workspace == x)
        return fail(FFN_ERR_INVALID, "ffn_decode_gemv_packed: workspace must not alias out, h or x");
    return hip_status(ffn::launch_decode_packed((uint16_t*)out, (uint16_t*)h, (uint16_t*)workspace,
                                                (const uint16_t*)x, w_gate, s_gate, w_up, s_up, w_down, s_down,
                                                (int)M, (int)C, (int)H, stream),
                      "ffn_decode_gemv_packed");
}

int64_t ffn_decode_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

ffn_status_t ffn_decode_gemv_packed_noalloc(void* out, void* h, const void* x, const uint8_t* w_gate,
                                            const float* s_gate, const uint8_t* w_up, const float* s_up,
                                            const uint8_t* w_down, const float* s_down, int64_t M, int64_t C,
                                            int64_t H, hipStream_t stream) {
    REQUIRE(s_gate);
    REQUIRE(s_up);
    REQUIRE(s_down);
    if (ffn_status_t st =
            check_decode("ffn_decode_gemv_packed_noalloc", out, h, x, w_gate, w_up, w_down, M, C, H, 1, 32))
        return st;
    const int64_t need = ffn::decode_packed_ws_elems((int)M, (int)C, (int)H) * 2;
    if (need > kNoAllocScratchBytes)
        return fail(FFN_ERR_UNSUPPORTED,
                    "ffn_decode_gemv_packed_noalloc: M = %lld, C = %lld, H = %lld need %lld bytes of workspace, "
                    "more than the %lld of the built-in scratch (use ffn_decode_gemv_packed)",
                    (long long)M, (long long)C, (long long)H, (long long)need, (long long)kNoAllocScratchBytes);
    if (M == 0) return FFN_OK;
    void* ws = nullptr;
    if (ffn_status_t st = hip_status(scratch_of_current_device(&ws), "ffn_decode_gemv_packed_noalloc")) return st;
    return hip_status(ffn::launch_decode_packed((uint16_t*)out, (uint16_t*)h, (uint16_t*)ws, (const uint16_t*)x,
                                                w_gate, s_gate, w_up, s_up, w_down, s_down, (int)M, (int)C, (int)H,
                                                stream),
                      "ffn_decode_gemv_packed_noalloc");
}

// ----------------------------------------------------------------------------- backward

ffn_status_t ffn_matmul_tn(void* out, const void* a, const float* a_scale, const void* b, const float* b_scale,
                           ffn_dtype_t dtype, int flags, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(a);
    REQUIRE(b);
    NONNEG(M);
    NONNEG(N);
    NONNEG(K);
    if (dtype != FFN_BF16 && dtype != FFN_E4M3 && dtype != FFN_E5M2)
        return fail(FFN_ERR_INVALID, "ffn_matmul_tn: unknown dtype %d", (int)dtype);
    if (flags & ~(FFN_TN_ACCUMULATE | FFN_TN_TILE_GRID | FFN_TN_TILED))
        return fail(FFN_ERR_INVALID, "ffn_matmul_tn: unknown flags 0x%x", (unsigned)flags);
    const bool fp8 = dtype != FFN_BF16;
    const bool tiled = (flags & FFN_TN_TILED) != 0;
    if (fp8) {
        REQUIRE(a_scale);
        REQUIRE(b_scale);
    }
    if (tiled && !fp8) return fail(FFN_ERR_UNSUPPORTED, "ffn_matmul_tn: tiled operands are FP8 codes");
    const int elt = fp8 ? 1 : 2;
    if (ffn_status_t st = check_gemm_dims("ffn_matmul_tn", M, K, N, elt)) return st;
    if (tiled && tiled_bytes(M, K) >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "ffn_matmul_tn: an operand exceeds 4 GiB");
    ALIGNED(out);
    ALIGNED(a);
    ALIGNED(b);
    if (out == a || out == b) return fail(FFN_ERR_INVALID, "ffn_matmul_tn: out must not alias an operand");
    return hip_status(ffn::launch_gemm(out, nullptr, a, a_scale, b, b_scale, fp8, false, M, (int)K, (int)N, stream,
                                       nullptr, nullptr, (flags & FFN_TN_ACCUMULATE) != 0, dtype == FFN_E5M2, nullptr,
                                       (flags & FFN_TN_TILE_GRID) != 0, true, tiled),
                      "ffn_matmul_tn");
}

static ffn_status_t matmul_tn_swiglu_bwd_entry(const char* fn, void* dgu, float* absmax, const void* a,
                                               const float* a_scale, const void* b, const float* b_scale,
                                               const void* gu, ffn_dtype_t dtype, int flags, int64_t M, int64_t H,
                                               int64_t K, hipStream_t stream, bool clear_absmax) {
    if (!dgu) return fail(FFN_ERR_INVALID, "%s: dgu is NULL", fn);
    if (!a) return fail(FFN_ERR_INVALID, "%s: a is NULL", fn);
    if (!b) return fail(FFN_ERR_INVALID, "%s: b is NULL", fn);
    if (!gu) return fail(FFN_ERR_INVALID, "%s: gu is NULL", fn);
    if (M < 0 || H < 0 || K < 0) return fail(FFN_ERR_INVALID, "%s: negative size", fn);
    if (dtype != FFN_BF16 && dtype != FFN_E4M3 && dtype != FFN_E5M2)
        return fail(FFN_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dtype);
    if (flags & ~(FFN_TN_TILE_GRID | FFN_TN_TILED))
        return fail(FFN_ERR_INVALID, "%s: unknown flags 0x%x", fn, (unsigned)flags);
    const bool fp8 = dtype != FFN_BF16;
    const bool tiled = (flags & FFN_TN_TILED) != 0;
    if (fp8 && !a_scale) return fail(FFN_ERR_INVALID, "%s: a_scale is NULL", fn);
    if (fp8 && !b_scale) return fail(FFN_ERR_INVALID, "%s: b_scale is NULL", fn);
    if (tiled && !fp8) return fail(FFN_ERR_UNSUPPORTED, "%s: tiled operands are FP8 codes", fn);
    if (ffn_status_t st = check_gemm_dims(fn, M, K, H, fp8 ? 1 : 2)) return st;
    if (tiled && tiled_bytes(M, K) >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "%s: an operand exceeds 4 GiB", fn);
    if (H > kMaxDim / 2) return fail(FFN_ERR_UNSUPPORTED, "%s: H = %lld too large", fn, (long long)H);
    if (misaligned(dgu) || misaligned(a) || misaligned(b) || misaligned(gu))
        return fail(FFN_ERR_UNSUPPORTED, "%s: a buffer is not 16-byte aligned", fn);
    if (dgu == a || dgu == b) return fail(FFN_ERR_INVALID, "%s: dgu must not alias a or b", fn);
    if (absmax && (absmax == a_scale || absmax == b_scale))
        return fail(FFN_ERR_INVALID, "%s: absmax must not alias a_scale or b_scale", fn);
    return hip_status(ffn::launch_gemm(dgu, absmax, a, a_scale, b, b_scale, fp8, false, M, (int)K, (int)H, stream,
                                       nullptr, nullptr, false, dtype == FFN_E5M2, gu, (flags & FFN_TN_TILE_GRID) != 0,
                                       clear_absmax, tiled),
                      fn);
}

ffn_status_t ffn_matmul_tn_swiglu_bwd(void* dgu, float* absmax, const void* a, const float* a_scale, const void* b,
                                      const float* b_scale, const void* gu, ffn_dtype_t dtype, int flags, int64_t M,
                                      int64_t H, int64_t K, hipStream_t stream) {
    return matmul_tn_swiglu_bwd_entry("ffn_matmul_tn_swiglu_bwd", dgu, absmax, a, a_scale, b, b_scale, gu, dtype,
                                      flags, M, H, K, stream, true);
}

ffn_status_t ffn_matmul_tn_swiglu_bwd_acc(void* dgu, float* absmax, const void* a, const float* a_scale,
                                          const void* b, const float* b_scale, const void* gu, ffn_dtype_t dtype,
                                          int flags, int64_t M, int64_t H, int64_t K, hipStream_t stream) {
    REQUIRE(absmax);
    return matmul_tn_swiglu_bwd_entry("ffn_matmul_tn_swiglu_bwd_acc", dgu, absmax, a, a_scale, b, b_scale, gu,
                                      dtype, flags, M, H, K, stream, false);
}

static ffn_status_t check_transpose(const char* fn, const void* out, const void* in, int64_t rows, int64_t cols,
                                    int64_t ld_out) {
    if (rows < 0 || cols < 0 || ld_out < 0) return fail(FFN_ERR_INVALID, "%s: negative size", fn);
    if (ld_out < rows) return fail(FFN_ERR_INVALID, "%s: ld_out = %lld < rows = %lld", fn, (long long)ld_out,
                                   (long long)rows);
    if (cols % 16 != 0 || ld_out % 16 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "%s: cols and ld_out must be multiples of 16", fn);
    if (cols > kMaxDim || ld_out > ((int64_t)65535 * 64))
        return fail(FFN_ERR_UNSUPPORTED, "%s: cols or ld_out too large", fn);
    if (misaligned(out) || misaligned(in)) return fail(FFN_ERR_UNSUPPORTED, "%s: a buffer is not 16-byte aligned", fn);
    if (out == in) return fail(FFN_ERR_INVALID, "%s: out must not alias in", fn);
    return FFN_OK;
}

ffn_status_t ffn_transpose(void* out, const void* in, int64_t rows, int64_t cols, int64_t ld_out, int elt_bytes,
                           hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(in);
    if (elt_bytes != 1 && elt_bytes != 2)
        return fail(FFN_ERR_INVALID, "ffn_transpose: element size %d (need 1 or 2)", elt_bytes);
    if (ffn_status_t st = check_transpose("ffn_transpose", out, in, rows, cols, ld_out)) return st;
    return hip_status(ffn::launch_transpose(out, nullptr, nullptr, nullptr, in, rows, (int)cols, ld_out, elt_bytes,
                                            elt_bytes, stream),
                      "ffn_transpose");
}

// The tiled output of a transposing call: rows of ld_out bytes (and, for the
// row-layout codes q, of cols bytes), whole 64-row groups within 32-bit
// offsets of one GEMM operand.
static ffn_status_t check_tiled_transpose(const char* fn, int64_t rows, int64_t cols, int64_t ld_out) {
    if (ld_out % 64 != 0 || cols % 64 != 0)
        return fail(FFN_ERR_UNSUPPORTED, "%s: cols and ld_out must be multiples of 64", fn);
    if (tiled_bytes(cols, ld_out) >= ((int64_t)1 << 32) || tiled_bytes(rows, cols) >= ((int64_t)1 << 32))
        return fail(FFN_ERR_UNSUPPORTED, "%s: an output exceeds 4 GiB", fn);
    return FFN_OK;
}

ffn_status_t ffn_transpose_tiled(uint8_t* out, const uint8_t* in, int64_t rows, int64_t cols, int64_t ld_out,
                                 hipStream_t stream) {
    REQUIRE(out);
    REQUIRE(in);
    if (ffn_status_t st = check_transpose("ffn_transpose_tiled", out, in, rows, cols, ld_out)) return st;
    if (ffn_status_t st = check_tiled_transpose("ffn_transpose_tiled", rows, cols, ld_out)) return st;
    return hip_status(ffn::launch_transpose(out, nullptr, nullptr, nullptr, in, rows, (int)cols, ld_out, 1, 1, stream,
                                            false, nullptr, true),
                      "ffn_transpose_tiled");
}

static ffn_status_t quant_transpose_entry(const char* fn, uint8_t* q_t, uint8_t* q, float* scale, const void* x,
                                          const float* absmax, float* clear, ffn_dtype_t code_dtype, int64_t rows,
                                          int64_t cols, int64_t ld_out, hipStream_t stream, bool tiled = false) {
    if (!q_t) return fail(FFN_ERR_INVALID, "%s: q_t is NULL", fn);
    if (!scale) return fail(FFN_ERR_INVALID, "%s: scale is NULL", fn);
    if (!x) return fail(FFN_ERR_INVALID, "%s: x is NULL", fn);
    if (!absmax) return fail(FFN_ERR_INVALID, "%s: absmax is NULL", fn);
    if (code_dtype != FFN_E4M3 && code_dtype != FFN_E5M2)
        return fail(FFN_ERR_INVALID, "%s: code dtype %d (need FFN_E4M3 or FFN_E5M2)", fn, (int)code_dtype);
    if (ffn_status_t st = check_transpose(fn, q_t, x, rows, cols, ld_out)) return st;
    if (misaligned(q)) return fail(FFN_ERR_UNSUPPORTED, "%s: q is not 16-byte aligned", fn);
    if (q && (q == q_t || (const void*)q == x)) return fail(FFN_ERR_INVALID, "%s: q must not alias q_t or x", fn);
    // every block reads *absmax while the first one writes *scale (and *clear)
    if ((const float*)scale == absmax) return fail(FFN_ERR_INVALID, "%s: scale and absmax alias", fn);
    if (clear && ((const float*)clear == absmax || clear == scale))
        return fail(FFN_ERR_INVALID, "%s: clear must not alias absmax or scale", fn);
    if (tiled)
        if (ffn_status_t st = check_tiled_transpose(fn, rows, cols, ld_out)) return st;
    return hip_status(ffn::launch_transpose(q_t, q, scale, absmax, x, rows, (int)cols, ld_out, 2, 1, stream,
                                            code_dtype == FFN_E5M2, clear, tiled),
                      fn);
}

ffn_status_t ffn_quant_transpose(uint8_t* q_t, uint8_t* q, float* scale, const void* x, const float* absmax,
                                 ffn_dtype_t code_dtype, int64_t rows, int64_t cols, int64_t ld_out,
                                 hipStream_t stream) {
    return quant_transpose_entry("ffn_quant_transpose", q_t, q, scale, x, absmax, nullptr, code_dtype, rows, cols,
                                 ld_out, stream);
}

ffn_status_t ffn_quant_transpose_clear(uint8_t* q_t, uint8_t* q, float* scale, const void* x, const float* absmax,
                                       float* clear, ffn_dtype_t code_dtype, int64_t rows, int64_t cols,
                                       int64_t ld_out, hipStream_t stream) {
    REQUIRE(clear);
    return quant_transpose_entry("ffn_quant_transpose_clear", q_t, q, scale, x, absmax, clear, code_dtype, rows,
                                 cols, ld_out, stream);
}

ffn_status_t ffn_quant_transpose_tiled(uint8_t* q_t, uint8_t* q, float* scale, const void* x, const float* absmax,
                                       float* clear, ffn_dtype_t code_dtype, int64_t rows, int64_t cols,
                                       int64_t ld_out, hipStream_t stream) {
    return quant_transpose_entry("ffn_quant_transpose_tiled", q_t, q, scale, x, absmax, clear, code_dtype, rows,
                                 cols, ld_out, stream, true);
}

static ffn_status_t swiglu_bwd_entry(const char* fn, void* dgu, float* absmax, const void* dh, const void* gu,
                                     int64_t N, int64_t H, hipStream_t stream, bool clear_absmax) {
    if (!dgu) return fail(FFN_ERR_INVALID, "%s: dgu is NULL", fn);
    if (!dh) return fail(FFN_ERR_INVALID, "%s: dh is NULL", fn);
    if (!gu) return fail(FFN_ERR_INVALID, "%s: gu is NULL", fn);
    if (N < 0 || H < 0) return fail(FFN_ERR_INVALID, "%s: negative size", fn);
    if (H < 8 || H % 8 != 0 || H > kMaxDim)
        return fail(FFN_ERR_UNSUPPORTED, "%s: H = %lld (need H %% 8 == 0)", fn, (long long)H);
    if (N * H > ((int64_t)1 << 36)) return fail(FFN_ERR_UNSUPPORTED, "%s: tensor too large", fn);
    if (misaligned(dgu) || misaligned(dh) || misaligned(gu))
        return fail(FFN_ERR_UNSUPPORTED, "%s: a buffer is not 16-byte aligned", fn);
    if (dgu == dh) return fail(FFN_ERR_INVALID, "%s: dgu must not alias dh", fn);
    return hip_status(ffn::launch_swiglu_bwd((uint16_t*)dgu, absmax, (const uint16_t*)dh, (const uint16_t*)gu, N,
                                             (int)H, stream, clear_absmax),
                      fn);
}

ffn_status_t ffn_swiglu_bwd(void* dgu, float* absmax, const void* dh, const void* gu, int64_t N, int64_t H,
                            hipStream_t stream) {
    return swiglu_bwd_entry("ffn_swiglu_bwd", dgu, absmax, dh, gu, N, H, stream, true);
}

ffn_status_t ffn_swiglu_bwd_acc(void* dgu, float* absmax, const void* dh, const void* gu, int64_t N, int64_t H,
                                hipStream_t stream) {
    REQUIRE(absmax);
    return swiglu_bwd_entry("ffn_swiglu_bwd_acc", dgu, absmax, dh, gu, N, H, stream, false);
}

int64_t ffn_rmsnorm_bwd_scratch_bytes(int64_t N, int64_t C) {
    if (N < 0 || C < 0 || C > 8192) return -1;
    return ffn::rmsnorm_bwd_scratch_floats(N, (int)C) * (int64_t)sizeof(float);
}

static ffn_status_t rmsnorm_bwd_entry(const char* fn, void* dinp, float* dweight, float* scratch,
                                      const void* dresidual, const void* dy, const void* r, const void* weight,
                                      const float* rstd, float* absmax, float* clear, int64_t N, int64_t C,
                                      hipStream_t stream, bool clear_absmax) {
    if (!dinp) return fail(FFN_ERR_INVALID, "%s: dinp is NULL", fn);
    if (!dweight) return fail(FFN_ERR_INVALID, "%s: dweight is NULL", fn);
    if (!scratch) return fail(FFN_ERR_INVALID, "%s: scratch is NULL", fn);
    if (!dresidual) return fail(FFN_ERR_INVALID, "%s: dresidual is NULL", fn);
    if (!dy) return fail(FFN_ERR_INVALID, "%s: dy is NULL", fn);
    if (!r) return fail(FFN_ERR_INVALID, "%s: r is NULL", fn);
    if (!weight) return fail(FFN_ERR_INVALID, "%s: weight is NULL", fn);
    if (!rstd) return fail(FFN_ERR_INVALID, "%s: rstd is NULL", fn);
    if (N < 0 || C < 0) return fail(FFN_ERR_INVALID, "%s: negative size", fn);
    if (C < 8 || C % 8 != 0 || C > 8192)
        return fail(FFN_ERR_UNSUPPORTED, "%s: C = %lld (need C %% 8 == 0, C <= 8192)", fn, (long long)C);
    if (N > ((int64_t)1 << 31)) return fail(FFN_ERR_UNSUPPORTED, "%s: N too large", fn);
    if (misaligned(dinp) || misaligned(dweight) || misaligned(scratch) || misaligned(dresidual) || misaligned(dy) ||
        misaligned(r) || misaligned(weight))
        return fail(FFN_ERR_UNSUPPORTED, "%s: a buffer is not 16-byte aligned", fn);
    if (dinp == dy || dinp == r) return fail(FFN_ERR_INVALID, "%s: dinp must not alias dy or r", fn);
    if (clear && clear == absmax) return fail(FFN_ERR_INVALID, "%s: clear must not alias absmax", fn);
    return hip_status(ffn::launch_rmsnorm_bwd((uint16_t*)dinp, dweight, scratch, (const uint16_t*)dresidual,
                                              (const uint16_t*)dy, (const uint16_t*)r, (const uint16_t*)weight, rstd,
                                              absmax, N, (int)C, stream, clear_absmax, clear),
                      fn);
}

ffn_status_t ffn_rmsnorm_bwd(void* dinp, float* dweight, float* scratch, const void* dresidual, const void* dy,
                             const void* r, const void* weight, const float* rstd, float* absmax, int64_t N,
                             int64_t C, hipStream_t stream) {
    return rmsnorm_bwd_entry("ffn_rmsnorm_bwd", dinp, dweight, scratch, dresidual, dy, r, weight, rstd, absmax,
                             nullptr, N, C, stream, true);
}

ffn_status_t ffn_rmsnorm_bwd_acc(void* dinp, float* dweight, float* scratch, const void* dresidual, const void* dy,
                                 const void* r, const void* weight, const float* rstd, float* absmax, float* clear,
                                 int64_t N, int64_t C, hipStream_t stream) {
    REQUIRE(absmax);
    return rmsnorm_bwd_entry("ffn_rmsnorm_bwd_acc", dinp, dweight, scratch, dresidual, dy, r, weight, rstd, absmax,
                             clear, N, C, stream, false);
}

}  // extern "C"
