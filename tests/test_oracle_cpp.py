"""Pins of the C++ oracle (oracle/ffn_oracle.cpp, fp32 with a fixed 16-way
summation order) against the numpy oracle (an independent implementation,
exact fp64 sums, itself pinned by closed forms, brute force and torch), against
closed forms, and against exact results on inputs whose every partial sum is
exact in fp32.  CPU only."""

import numpy as np
import pytest

import oracle as O
from oracle import codecs as K
from oracle import cpp as P
from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import rel_err, ulp_diff


@pytest.fixture(scope="module", autouse=True)
def built():
    P.lib()


def _f32_of_bits(u32):
    return np.asarray(u32, np.uint32).view(np.float32)


def test_bf16_rounding_matches_the_numpy_codec():
    rng = np.random.default_rng(1)
    # every bf16 value, and the values half an ulp either side of each (ties
    # to even), plus random fp32 patterns and the edges
    b = np.arange(65536, dtype=np.uint32)
    tie = (b << 16) | 0x8000
    vals = np.concatenate([_f32_of_bits(b << 16), _f32_of_bits(tie), _f32_of_bits(tie + 1), _f32_of_bits(tie - 1),
                           _f32_of_bits(rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)),
                           np.array([3.4e38, -3.4e38, 1e-45, -0.0, 0.0, np.inf, -np.inf], np.float32)])
    got = P.bf16_round_f32(vals)
    want = K.f64_to_bf16_bits(vals.astype(np.float64))
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)          # NaN stays NaN (sign and payload unspecified)


def test_e4m3_codec_matches_the_numpy_codec():
    codes = np.arange(256, dtype=np.uint8)
    got, want = P.e4m3_decode(codes).astype(np.float64), K.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    vals = K.bf16_bits_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16)).astype(np.float32)
    for s in (1.0, 0.37, 448.0 / 3.0, 2.0 ** -7, 1e30):
        v = (vals * np.float32(s)).astype(np.float32)
        assert np.array_equal(P.e4m3_encode(v), K.e4m3_encode(v)), s
    # landmarks: 448 saturates, 2^-6 is the smallest normal, 2^-9 the smallest subnormal
    assert list(P.e4m3_encode(np.array([448, 500, 2 ** -6, 2 ** -9, 2 ** -10, -0.0], np.float32))) == \
        [0x7E, 0x7E, 0x08, 0x01, 0x00, 0x80]


@pytest.mark.parametrize("N,C,add", [(37, 384, True), (5, 4096, False), (64, 256, True), (3, 8, True)])
def test_rmsnorm_matches_numpy_and_closed_forms(N, C, add):
    d = W.block_inputs(N, C, 128, seed=N + C, outliers=True)
    inp, addend, w = d["inp"], d["addend"] if add else None, d["w_norm"]
    r, y, rstd, am = P.rmsnorm_fwd(inp, addend, w, 1e-5)
    r_n, y_n, rstd_n, am_n = O.rmsnorm_fwd(inp, addend, w, 1e-5)
    if add:
        assert np.array_equal(r, r_n)
    else:
        assert r is None
    # a sequential fp32 sum of C non-negative squares is within C 2^-24 of
    # the exact sum (relative); rstd = (sum / C + eps)^-1/2 moves by half of
    # that, plus a few roundings of the division, square root and reciprocal
    assert np.max(np.abs(rstd / rstd_n - 1)) < (C / 2 + 4) * 2.0 ** -24
    y_given, am_given = O.rms_apply(r_n if add else inp, rstd, w)  # the numpy oracle's fp32 products
    assert np.array_equal(y, y_given) and am == am_given
    assert ulp_diff(y, y_n).max() <= 1


def test_rmsnorm_closed_forms():
    N, C = 4, 1024
    x = W.normal_bf16((N, C), 3.0, 2, 1)
    ones = W.to_bf16_bits(np.ones(C, np.float32))
    _, y, rstd, _ = P.rmsnorm_fwd(x, None, ones, 0.0)
    yv = K.bf16_bits_to_f64(y)
    assert np.allclose(np.mean(yv * yv, axis=1), 1.0, atol=1e-2)   # unit RMS with unit weight, eps = 0
    z = np.zeros((2, C), np.uint16)
    _, y0, rstd0, am0 = P.rmsnorm_fwd(z, None, ones, 1e-5)
    assert np.all(y0 == 0) and am0 == 0
    assert np.allclose(rstd0, 1.0 / np.sqrt(np.float32(1e-5)), rtol=1e-6)


def test_quant_matches_numpy_bit_for_bit():
    x = W.block_inputs(300, 512, 128, seed=3, outliers=True)["inp"]
    for am in (None, np.float32(2.5), np.float32(0.0)):
        q, s, a = P.quant_absmax(x, am)
        qn, sn, an = O.quant_absmax(x, am)
        assert np.array_equal(q, qn) and s == sn and a == an
    # the largest element maps to +-448
    q, s, a = P.quant_absmax(x)
    assert np.max(P.e4m3_decode(q).astype(np.float64) * s) == pytest.approx(float(a), rel=1e-6)
    assert (q[np.unravel_index(np.argmax(np.abs(K.bf16_bits_to_f64(x))), x.shape)] & 0x7F) == 0x7E


def test_absmax_propagates_nan():
    x = W.normal_bf16((1000,), 1.0, 4, 1)
    x[321] = 0x7FC0
    assert np.isnan(P.absmax_of(x))
    q, s, a = P.quant_absmax(x)
    assert np.isnan(s) and np.all((q & 0x7F) == 0x7F)


def _int_bf16(shape, seed):
    return W.to_bf16_bits(np.random.default_rng(seed).integers(-4, 5, shape).astype(np.float32))


@pytest.mark.parametrize("N,K_,O_", [(37, 256, 48), (5, 1000, 130), (64, 4096, 32)])
def test_gemms_exact_on_integer_inputs(N, K_, O_):
    # every partial sum is an integer below 2^24: exact in fp32 in any order
    x, w = _int_bf16((N, K_), 1), _int_bf16((O_, K_), 2)
    assert np.array_equal(P.gemm_bf16(x, w), O.gemm_bf16(x, w))
    qx = K.e4m3_encode(np.random.default_rng(3).integers(-4, 5, (N, K_)).astype(np.float32))
    qw = K.e4m3_encode(np.random.default_rng(4).integers(-4, 5, (O_, K_)).astype(np.float32))
    assert np.array_equal(P.gemm_fp8(qx, 1.0, qw, 1.0), O.gemm_fp8(qx, np.float32(1), qw, np.float32(1)))


@pytest.mark.parametrize("N,K_,O_", [(37, 256, 48), (9, 3584, 130)])
def test_gemms_within_the_fp32_accumulation_bound(N, K_, O_):
    # each partial sum adds K/16 exact products, then four pairwise levels:
    # |error| <= (K/16 + 4) 2^-24 sum |a b|, plus the final bf16 rounding
    d = W.block_inputs(N, K_, O_, seed=7, w_std=0.0, outliers=True)
    x, w = d["inp"], d["w_gu"][:O_]
    xf, wf = K.bf16_bits_to_f64(x), K.bf16_bits_to_f64(w)
    exact, mag = xf @ wf.T, np.abs(xf) @ np.abs(wf).T
    got = K.bf16_bits_to_f64(P.gemm_bf16(x, w))
    gamma = (K_ / 16 + 4) * 2.0 ** -24
    assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) + gamma * mag * 1.01)
    qx, sx, _ = O.quant_absmax(x)
    qw, sw, _ = O.quant_absmax(w)
    ex8 = (K.e4m3_decode(qx) @ K.e4m3_decode(qw).T) * float(np.float32(sx * sw))
    mag8 = (np.abs(K.e4m3_decode(qx)) @ np.abs(K.e4m3_decode(qw)).T) * float(np.float32(sx * sw))
    got8 = K.bf16_bits_to_f64(P.gemm_fp8(qx, sx, qw, sw))
    assert np.all(np.abs(got8 - ex8) <= 2.0 ** -8 * np.abs(ex8) + (gamma + 2.0 ** -23) * mag8 * 1.01)


def test_gemm_summation_order_is_the_documented_one():
    # K = 32, one output: term 0 = 2^24, term 16 = 1 (both in partial sum 0)
    # and term 8 = -2^24 (partial sum 8).  Partial 0 = fl(2^24 + 1) = 2^24,
    # partial 8 = -2^24; the pairwise step adds partial 8 into partial 0: 0.
    # A sequential sum would give 1, the exact sum is 1.
    x = W.to_bf16_bits(np.ones((1, 32), np.float32))
    wv = np.zeros((1, 32), np.float32)
    wv[0, 0], wv[0, 16], wv[0, 8] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    assert K.bf16_bits_to_f64(P.gemm_bf16(x, W.to_bf16_bits(wv)))[0, 0] == 0.0
    # the same terms in partial sums 0, 1 and 2 are combined as
    # ((p0 + p1) + (p2 + p3)) ...: p0 + p1 = 2^24 + 1 -> 2^24, then + p2 = 0
    wv = np.zeros((1, 32), np.float32)
    wv[0, 0], wv[0, 1], wv[0, 2] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    # level 1: p0 += p8 ... (p8 = 0), so p0 = 2^24, p1 = 1, p2 = -2^24;
    # level 2: p0 += p4, p1 += p5, p2 += p6; level 3: p0 += p2 -> 0, p1 += p3;
    # level 4: p0 += p1 -> 1
    assert K.bf16_bits_to_f64(P.gemm_bf16(x, W.to_bf16_bits(wv)))[0, 0] == 1.0


def test_magnitude_products():
    d = W.block_inputs(20, 512, 64, seed=13, w_std=0.0)
    x, w = d["inp"], d["w_gu"]
    want = np.abs(K.bf16_bits_to_f64(x)) @ np.abs(K.bf16_bits_to_f64(w)).T
    assert np.allclose(P.gemm_abs_bf16(x, w), want, rtol=1e-5)
    qx, sx, _ = O.quant_absmax(x)
    qw, sw, _ = O.quant_absmax(w)
    want8 = (np.abs(K.e4m3_decode(qx)) @ np.abs(K.e4m3_decode(qw)).T) * float(np.float32(sx * sw))
    assert np.allclose(P.gemm_abs_fp8(qx, sx, qw, sw), want8, rtol=1e-5)


def test_swiglu_matches_numpy():
    gu = W.normal_bf16((64, 2 * 768), 2.0, 5, 2)
    h, am = P.swiglu(gu)
    hn, amn = O.swiglu(gu)
    assert ulp_diff(h, hn).max() <= 1 and np.mean(ulp_diff(h, hn) != 0) < 1e-2
    assert am == P.absmax_of(h)
    # silu(0) = 0: a zero gate gives h = 0 whatever u is
    z = gu.copy()
    z[:, :768] = 0
    assert np.all(K.bf16_bits_to_f64(P.swiglu(z)[0]) == 0)


@pytest.mark.parametrize("M,C,H", [(1, 256, 768), (16, 384, 512), (3, 1024, 256)])
def test_decode_matches_numpy(M, C, H):
    d = W.decode_inputs(M, C, H, seed=M + C + H)
    qg, sg = O.quant_rows(d["w_gate"])
    qu, su = O.quant_rows(d["w_up"])
    qd, sd = O.quant_rows(d["w_down"])
    y, h = P.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    y_n, h_n = O.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    assert rel_err(h, h_n) < 2e-2 and np.mean(h != h_n) < 2e-2
    assert rel_err(y, O.decode_down(h, qd, sd)) < 1e-2
    assert rel_err(y, y_n) < 3e-2


@pytest.mark.parametrize("fp8", [False, True])
def test_block_matches_numpy(fp8):
    d = W.block_inputs(96, 512, 384, seed=11, w_std=0.0, outliers=True)
    a = P.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=fp8)
    b = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=fp8)
    assert np.array_equal(a["residual"], b["residual"])
    assert rel_err(a["h"], b["h"]) < 3e-2
    assert rel_err(a["down"], b["down"]) < 3e-2
    assert rel_err(a["next_residual"], b["next_residual"]) < 3e-2
    # the closing residual is one rounding of r + down
    r = K.bf16_bits_to_f64(a["residual"])
    assert np.array_equal(a["next_residual"], K.f64_to_bf16_bits(r + K.bf16_bits_to_f64(a["down"])))


def test_thread_count_does_not_change_results():
    d = W.block_inputs(50, 256, 256, seed=12, w_std=0.0)
    one = P.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=True, nthreads=1)
    many = P.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=True, nthreads=7)
    for k in ("y", "rstd", "qy", "h", "qh", "down"):
        assert np.array_equal(one[k], many[k]), k


def test_cpu_info():
    model, logical, physical = P.cpu_info()
    assert logical >= 1 and 1 <= physical <= max(logical, 1024)
    assert isinstance(model, str)
