// Plain C++ oracle of the FFN block forward and its FP8 decode form.
// TEST INFRASTRUCTURE ONLY: built by oracle/cpp.py with the host compiler and
// used by tests/, the smoke check and the CPU baseline of the benchmark.  It
// shares no code with the HIP library and includes none of its headers.
//
// What it computes follows three pages: llmq llama_model.cpp
// (LLamaModel::_forward_block: fused_residual_rmsnorm_forward into LN2,
// forward_qmm with the [2H, C] up weight, swiglu_forward, forward_qmm with the
// [C, H] down weight; forward_qmm: quantize_with_abs_max, then the matmul
// scaled by the weight's and the input's scales), llmq llama_run_state.cpp
// (rstd fp32 [B, T]; e4m3 copies with an abs-max and a scale each) and metrale
// dense_ffn_decode.rs (DenseFfnLayer::forward, FP8 arm: w8a16_gemv_dual with
// per-row scales, silu_mul, w8a16_gemv).
//
// Arithmetic: fp32 throughout, every stored value rounded once to its storage
// type (bf16 activations, fp32 rstd and scales, e4m3 codes).  Dot products
// accumulate in fp32 in one fixed order: sixteen strided partial sums
// (partial j takes the terms k = j, j + 16, j + 32, ... in turn), combined
// pairwise (j + 8 into j, then j + 4, j + 2, j + 1).  Every product of two
// bf16 or e4m3 values is exact in fp32, so a fused multiply-add would give the
// same sums; the build turns contraction off all the same.  Threads split the
// output rows only, so results do not depend on the thread count.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <set>
#include <string>
#include <thread>
#include <utility>
#include <vector>

namespace {

// ---------------------------------------------------------------- codecs

// bf16 = the top 16 bits of an IEEE binary32.
float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Round an fp32 to bf16, to nearest with ties to even: add half of the
// dropped range (minus one when the kept part is even) and truncate.  A
// carry out of the mantissa raises the exponent, and past the largest finite
// value it gives infinity, as rounding requires.  A NaN becomes a quiet NaN
// with its sign.
uint16_t bf16_round(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    const uint32_t keep_odd = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + keep_odd) >> 16);
}

// e4m3 (OCP E4M3FN): sign, 4 exponent bits (bias 7), 3 mantissa bits; codes
// 0x7F and 0xFF are NaN; no infinities; largest finite 448.
float e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return std::nanf("");
    const float mag = e == 0 ? std::ldexp((float)m / 8.0f, -6) : std::ldexp(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

// Nearest e4m3 code, ties to the even code, magnitudes at or above 448
// saturated to 448, NaN to 0x7F with the sign bit, -0 to 0x80.
uint8_t e4m3_code(float v) {
    const uint8_t s = std::signbit(v) ? 0x80 : 0x00;
    if (std::isnan(v)) return s | 0x7F;
    const float a = std::fabs(v);
    if (a >= 448.0f) return s | 0x7E;
    if (a < std::ldexp(1.0f, -6)) {
        // subnormal grid 2^-9: codes 0 .. 8 (8 is the smallest normal, 0x08)
        return s | (uint8_t)std::nearbyint(a * 512.0f);
    }
    int ex;
    std::frexp(a, &ex);          // a = f 2^ex, 0.5 <= f < 1
    int e = ex - 1;              // a = (1 + m/8) 2^e
    int m = (int)std::nearbyint((std::ldexp(a, -e) - 1.0f) * 8.0f);
    if (m == 8) {
        m = 0;
        e += 1;
    }
    return s | (uint8_t)(((e + 7) << 3) | m);
}

// ---------------------------------------------------------------- helpers

// The fixed-order fp32 dot product described at the top of the file.
float dot16(const float* a, const float* b, int64_t K) {
    float acc[16];
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
    int64_t k = 0;
    for (; k + 16 <= K; k += 16)
        for (int j = 0; j < 16; ++j) acc[j] += a[k + j] * b[k + j];
    for (int j = 0; k + j < K; ++j) acc[j] += a[k + j] * b[k + j];
    for (int w = 8; w >= 1; w >>= 1)
        for (int j = 0; j < w; ++j) acc[j] = acc[j] + acc[j + w];
    return acc[0];
}

// Run f(lo, hi) over [0, n) in chunks of `grain` on `threads` threads.
template <class F>
void parallel_rows(int64_t n, int64_t grain, int threads, F f) {
    if (threads < 1) threads = 1;
    std::atomic<int64_t> next(0);
    auto work = [&]() {
        for (;;) {
            const int64_t lo = next.fetch_add(grain);
            if (lo >= n) break;
            f(lo, std::min(n, lo + grain));
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < threads; ++t) pool.emplace_back(work);
    work();
    for (auto& t : pool) t.join();
}

// dot16 of one row a against four rows b0..b3 at once (the loads of a are
// shared); each of the four sums takes exactly the operations, in exactly
// the order, that dot16 would.
void dot16x4(const float* __restrict a, const float* __restrict b0, const float* __restrict b1,
             const float* __restrict b2, const float* __restrict b3, int64_t K, float out[4]) {
    float c0[16], c1[16], c2[16], c3[16];
    for (int j = 0; j < 16; ++j) c0[j] = c1[j] = c2[j] = c3[j] = 0.0f;
    int64_t k = 0;
    for (; k + 16 <= K; k += 16)
        for (int j = 0; j < 16; ++j) {
            const float av = a[k + j];
            c0[j] += av * b0[k + j];
            c1[j] += av * b1[k + j];
            c2[j] += av * b2[k + j];
            c3[j] += av * b3[k + j];
        }
    for (int j = 0; k + j < K; ++j) {
        const float av = a[k + j];
        c0[j] += av * b0[k + j];
        c1[j] += av * b1[k + j];
        c2[j] += av * b2[k + j];
        c3[j] += av * b3[k + j];
    }
    float* c[4] = {c0, c1, c2, c3};
    for (int r = 0; r < 4; ++r) {
        for (int w = 8; w >= 1; w >>= 1)
            for (int j = 0; j < w; ++j) c[r][j] = c[r][j] + c[r][j + w];
        out[r] = c[r][0];
    }
}

// out[n, o] = dot16(x[n, :], w[o, :]) for fp32 operand rows; the outputs of
// one block of token rows are computed weight block by weight block, so a
// block of weight rows is reused from cache (each output's sum is unchanged).
template <class Store>
void matmul_nt(const float* x, const float* w, int64_t N, int64_t K, int64_t O, int threads, Store store) {
    constexpr int64_t kRowBlk = 16, kWBlk = 64;
    parallel_rows(N, kRowBlk, threads, [&](int64_t n0, int64_t n1) {
        for (int64_t o0 = 0; o0 < O; o0 += kWBlk) {
            const int64_t o1 = std::min(O, o0 + kWBlk);
            for (int64_t n = n0; n < n1; ++n) {
                int64_t o = o0;
                for (; o + 4 <= o1; o += 4) {
                    float v[4];
                    dot16x4(x + n * K, w + o * K, w + (o + 1) * K, w + (o + 2) * K, w + (o + 3) * K, K, v);
                    for (int r = 0; r < 4; ++r) store(n, o + r, v[r]);
                }
                for (; o < o1; ++o) store(n, o, dot16(x + n * K, w + o * K, K));
            }
        }
    });
}

std::vector<float> bf16_to_f32(const uint16_t* b, int64_t n, int threads) {
    std::vector<float> f((size_t)n);
    parallel_rows(n, 1 << 16, threads, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo; i < hi; ++i) f[(size_t)i] = bf16_value(b[i]);
    });
    return f;
}

std::vector<float> e4m3_to_f32(const uint8_t* q, int64_t n, int threads) {
    float table[256];
    for (int c = 0; c < 256; ++c) table[c] = e4m3_value((uint8_t)c);
    std::vector<float> f((size_t)n);
    parallel_rows(n, 1 << 16, threads, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo; i < hi; ++i) f[(size_t)i] = table[q[i]];
    });
    return f;
}

float silu_times(float g, float u) { return (g / (1.0f + std::exp(-g))) * u; }

// max |x| that propagates NaN (a NaN element makes the result NaN).
float absmax_update(float m, float v) {
    const float a = std::fabs(v);
    if (std::isnan(a) || std::isnan(m)) return std::nanf("");
    return a > m ? a : m;
}

}  // namespace

extern "C" {

// bf16 and e4m3 codecs over arrays (for the pins of the codecs themselves).
void ffo_bf16_round(uint16_t* out, const float* v, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
}
void ffo_e4m3_encode(uint8_t* out, const float* v, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_code(v[i]);
}
void ffo_e4m3_decode(float* out, const uint8_t* q, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(q[i]);
}

// Fused residual add + RMSNorm (llmq llama_model.cpp, _forward_block,
// fused_residual_rmsnorm_forward; without an addend, rmsnorm_forward):
//   r = bf16(inp + addend)              (r = inp without an addend)
//   ss = sum_j r_j^2                    (fp32, j in order)
//   rstd = 1 / sqrt(ss / C + eps)       (fp32)
//   y = bf16((r * rstd) * w)            (two fp32 products)
//   absmax = max |y| over the stored y
// res may be null (then r is not stored); absmax may be null.
void ffo_rmsnorm_fwd(uint16_t* y, float* rstd, uint16_t* res, float* absmax, const uint16_t* inp,
                     const uint16_t* addend, const uint16_t* w, float eps, int64_t N, int64_t C, int threads) {
    std::vector<float> row_max((size_t)std::max<int64_t>(N, 1), 0.0f);
    parallel_rows(N, 16, threads, [&](int64_t n0, int64_t n1) {
        std::vector<uint16_t> r((size_t)C);
        for (int64_t n = n0; n < n1; ++n) {
            for (int64_t j = 0; j < C; ++j) {
                const uint16_t a = inp[n * C + j];
                r[(size_t)j] = addend ? bf16_round(bf16_value(a) + bf16_value(addend[n * C + j])) : a;
            }
            float ss = 0.0f;
            for (int64_t j = 0; j < C; ++j) ss += bf16_value(r[(size_t)j]) * bf16_value(r[(size_t)j]);
            const float rs = 1.0f / std::sqrt(ss / (float)C + eps);
            rstd[n] = rs;
            float m = 0.0f;
            for (int64_t j = 0; j < C; ++j) {
                const uint16_t yb = bf16_round((bf16_value(r[(size_t)j]) * rs) * bf16_value(w[j]));
                y[n * C + j] = yb;
                m = absmax_update(m, bf16_value(yb));
                if (res) res[n * C + j] = r[(size_t)j];
            }
            row_max[(size_t)n] = m;
        }
    });
    if (absmax) {
        float m = 0.0f;
        for (int64_t n = 0; n < N; ++n) m = absmax_update(m, row_max[(size_t)n]);
        *absmax = m;
    }
}

// max |x| over a bf16 tensor (llmq _forward_block, abs_max); NaN propagates.
float ffo_absmax(const uint16_t* x, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) m = absmax_update(m, bf16_value(x[i]));
    return m;
}

// Per-tensor e4m3 quantisation with a given abs-max (llmq forward_qmm,
// quantize_with_abs_max): scale = absmax / 448 and inv = 448 / absmax, both
// fp32 quotients (1 and 1 when absmax == 0); q = e4m3(x * inv), the product
// in fp32.  Returns the scale.
float ffo_quant(uint8_t* q, const uint16_t* x, int64_t n, float absmax, int threads) {
    const float scale = absmax == 0.0f ? 1.0f : absmax / 448.0f;
    const float inv = absmax == 0.0f ? 1.0f : 448.0f / absmax;
    parallel_rows(n, 1 << 16, threads, [&](int64_t lo, int64_t hi) {
        for (int64_t i = lo; i < hi; ++i) q[i] = e4m3_code(bf16_value(x[i]) * inv);
    });
    return scale;
}

// bf16 GEMM: out[n, o] = bf16(sum_k x[n, k] w[o, k]) (llmq forward_qmm,
// matmul TN with bf16 operands).
void ffo_gemm_bf16(uint16_t* out, const uint16_t* x, const uint16_t* w, int64_t N, int64_t K, int64_t O,
                   int threads) {
    const std::vector<float> xf = bf16_to_f32(x, N * K, threads), wf = bf16_to_f32(w, O * K, threads);
    matmul_nt(xf.data(), wf.data(), N, K, O, threads,
              [&](int64_t n, int64_t o, float v) { out[n * O + o] = bf16_round(v); });
}

// FP8 GEMM: out[n, o] = bf16(sum_k dec(qx[n, k]) dec(qw[o, k]) * (sx * sw)),
// the two scales multiplied once in fp32 (llmq forward_qmm with weight.scale()
// and inp.Quant.scale()).
void ffo_gemm_fp8(uint16_t* out, const uint8_t* qx, float sx, const uint8_t* qw, float sw, int64_t N, int64_t K,
                  int64_t O, int threads) {
    const std::vector<float> xf = e4m3_to_f32(qx, N * K, threads), wf = e4m3_to_f32(qw, O * K, threads);
    const float s = sx * sw;
    matmul_nt(xf.data(), wf.data(), N, K, O, threads,
              [&](int64_t n, int64_t o, float v) { out[n * O + o] = bf16_round(v * s); });
}

// Magnitude products for error bounds: out[n, o] = sum_k |x[n, k]| |w[o, k]|
// (times |sx sw| for e4m3 operands), in fp32 (a bound needs no more).
void ffo_gemm_abs_bf16(float* out, const uint16_t* x, const uint16_t* w, int64_t N, int64_t K, int64_t O,
                       int threads) {
    std::vector<float> xf = bf16_to_f32(x, N * K, threads), wf = bf16_to_f32(w, O * K, threads);
    for (auto& v : xf) v = std::fabs(v);
    for (auto& v : wf) v = std::fabs(v);
    matmul_nt(xf.data(), wf.data(), N, K, O, threads, [&](int64_t n, int64_t o, float v) { out[n * O + o] = v; });
}
void ffo_gemm_abs_fp8(float* out, const uint8_t* qx, float sx, const uint8_t* qw, float sw, int64_t N, int64_t K,
                      int64_t O, int threads) {
    std::vector<float> xf = e4m3_to_f32(qx, N * K, threads), wf = e4m3_to_f32(qw, O * K, threads);
    for (auto& v : xf) v = std::fabs(v);
    for (auto& v : wf) v = std::fabs(v);
    const float s = std::fabs(sx * sw);
    matmul_nt(xf.data(), wf.data(), N, K, O, threads, [&](int64_t n, int64_t o, float v) { out[n * O + o] = v * s; });
}

// SwiGLU on the [N, 2H] up-projection output (llmq _forward_block,
// swiglu_forward): h[n, j] = bf16((g / (1 + exp(-g))) * u), g = gu[n, j],
// u = gu[n, H + j] (gate columns first); returns max |h|.
float ffo_swiglu(uint16_t* h, const uint16_t* gu, int64_t N, int64_t H, int threads) {
    std::vector<float> row_max((size_t)std::max<int64_t>(N, 1), 0.0f);
    parallel_rows(N, 16, threads, [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n) {
            float m = 0.0f;
            for (int64_t j = 0; j < H; ++j) {
                const uint16_t hb =
                    bf16_round(silu_times(bf16_value(gu[n * 2 * H + j]), bf16_value(gu[n * 2 * H + H + j])));
                h[n * H + j] = hb;
                m = absmax_update(m, bf16_value(hb));
            }
            row_max[(size_t)n] = m;
        }
    });
    float m = 0.0f;
    for (int64_t n = 0; n < N; ++n) m = absmax_update(m, row_max[(size_t)n]);
    return m;
}

// The FP8 decode FFN, split-SiLU arm (metrale dense_ffn_decode.rs,
// DenseFfnLayer::forward, FP8 arm):
//   g[m, n] = bf16(sg[n] * sum_k dec(wg[n, k]) x[m, k]),  u likewise
//   h[m, n] = bf16(silu(g) * u)
//   y[m, c] = bf16(sd[c] * sum_n dec(wd[c, n]) h[m, n])
void ffo_decode(uint16_t* y, uint16_t* h, const uint16_t* x, const uint8_t* wg, const float* sg, const uint8_t* wu,
                const float* su, const uint8_t* wd, const float* sd, int64_t M, int64_t C, int64_t H, int threads) {
    const std::vector<float> xf = bf16_to_f32(x, M * C, threads);
    const std::vector<float> gf = e4m3_to_f32(wg, H * C, threads), uf = e4m3_to_f32(wu, H * C, threads);
    std::vector<float> g((size_t)(M * H)), u((size_t)(M * H));
    matmul_nt(xf.data(), gf.data(), M, C, H, threads,
              [&](int64_t m, int64_t n, float v) { g[(size_t)(m * H + n)] = bf16_value(bf16_round(sg[n] * v)); });
    matmul_nt(xf.data(), uf.data(), M, C, H, threads,
              [&](int64_t m, int64_t n, float v) { u[(size_t)(m * H + n)] = bf16_value(bf16_round(su[n] * v)); });
    for (int64_t i = 0; i < M * H; ++i) h[i] = bf16_round(silu_times(g[(size_t)i], u[(size_t)i]));
    const std::vector<float> hf = bf16_to_f32(h, M * H, threads), df = e4m3_to_f32(wd, C * H, threads);
    matmul_nt(hf.data(), df.data(), M, H, C, threads,
              [&](int64_t m, int64_t c, float v) { y[m * C + c] = bf16_round(sd[c] * v); });
}

// Host description for the CPU baseline: the CPU model string, the logical
// CPUs this process may run on, and the physical cores among them (distinct
// (package, core) pairs in /proc/cpuinfo).
void ffo_cpu_info(char* model, int model_len, int* logical, int* physical) {
    *logical = (int)std::thread::hardware_concurrency();
    std::ifstream f("/proc/cpuinfo");
    std::string line, name;
    std::set<std::pair<int, int>> cores;
    int phys = -1, core = -1;
    while (std::getline(f, line)) {
        const auto colon = line.find(':');
        if (colon == std::string::npos) {
            if (phys >= 0 || core >= 0) cores.insert({phys, core});
            phys = core = -1;
            continue;
        }
        std::string key = line.substr(0, colon), val = line.substr(colon + 1);
        while (!key.empty() && (key.back() == ' ' || key.back() == '\t')) key.pop_back();
        while (!val.empty() && val.front() == ' ') val.erase(0, 1);
        if (key == "model name" && name.empty()) name = val;
        if (key == "physical id") phys = std::atoi(val.c_str());
        if (key == "core id") core = std::atoi(val.c_str());
    }
    if (phys >= 0 || core >= 0) cores.insert({phys, core});
    *physical = cores.empty() ? *logical : (int)cores.size();
    std::snprintf(model, (size_t)model_len, "%s", name.c_str());
}

}  // extern "C"
