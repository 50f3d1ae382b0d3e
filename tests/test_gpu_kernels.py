"""GPU parity of each HIP kernel against the CPU oracle, through the C ABI.

Bit-exact where the result is unique (residual sums, abs-maxes, e4m3 codes given
the same input and abs-max, GEMMs on integer-valued inputs, fused vs unfused
SwiGLU); within a stated tolerance where fp32 summation order or the hardware
exp/rsqrt decides the last bit.  Shapes span several tiles and ragged tails.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import codecs as K
from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import (say, dev_bf16, dev_u8, dev_f32, host_bits, host_u8, host_f32, empty_bf16,
                            empty_f32, empty_u8, rel_err, ulp_diff, within_dot_bound)


def _exact_and_mag(a, b, s=1.0):
    """Exact fp64 product a @ b^T times s, and sum_k |a_k b_k| times |s|."""
    return (a @ b.T) * s, (np.abs(a) @ np.abs(b).T) * abs(s)

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_ffn_block_residual_amd as F
    return F


# ----------------------------------------------------------------------------- RMSNorm

RMS_SHAPES = [(64, 256, True), (37, 384, True), (300, 4096, True), (129, 3584, True), (5, 8192, False),
              (3, 16384, True), (1, 8, True), (77, 1000, False), (4, 12288, False), (2, 16384, False)]


@pytest.mark.parametrize("N,C,add", RMS_SHAPES)
def test_rmsnorm(F, N, C, add):
    say(f"rmsnorm N={N} C={C} add={add}")
    d = W.block_inputs(N, C, 128, seed=N * 7 + C, outliers=(C == 4096))
    inp, addend, w = d["inp"], d["addend"] if add else None, d["w_norm"]
    y, rstd, am = empty_bf16(N, C), empty_f32(N), empty_f32(1)
    res = empty_bf16(N, C) if add else None
    F.ffn_rmsnorm_fwd(y, rstd, res, am, dev_bf16(inp), dev_bf16(addend) if add else None, dev_bf16(w),
                      1e-5, N, C)
    torch.cuda.synchronize()
    r_ref, y_ref, rstd_ref, am_ref = O.rmsnorm_fwd(inp, addend, w, 1e-5)
    if add:
        assert np.array_equal(host_bits(res), r_ref)                       # unique: bit-exact
    g_rstd = host_f32(rstd)
    assert np.max(np.abs(g_rstd / rstd_ref - 1)) < 1e-5
    gy = host_bits(y)
    # y given the GPU's own rstd: both take (r * rstd) * w as two fp32
    # products and round once to bf16, so y is unique
    y_cond, _ = O.rms_apply(r_ref if add else inp, g_rstd, w)
    assert np.array_equal(gy, y_cond)
    assert rel_err(gy, y_ref) < 2e-2
    assert host_f32(am)[0] == np.max(np.abs(K.bf16_bits_to_f64(gy)))  # abs-max of what was stored


def test_rmsnorm_in_place_and_empty(F):
    N, C = 50, 2048
    say(f"rmsnorm in place N={N} C={C}")
    d = W.block_inputs(N, C, 128, seed=3)
    inp = dev_bf16(d["inp"])
    addend = dev_bf16(d["addend"])
    res, rstd, am = empty_bf16(N, C), empty_f32(N), empty_f32(1)
    F.ffn_rmsnorm_fwd(addend, rstd, res, am, inp, addend, dev_bf16(d["w_norm"]), 1e-5, N, C)  # y overwrites addend
    torch.cuda.synchronize()
    r_ref, y_ref, _, am_ref = O.rmsnorm_fwd(d["inp"], d["addend"], d["w_norm"], 1e-5)
    assert np.array_equal(host_bits(res), r_ref)
    assert rel_err(host_bits(addend), y_ref) < 2e-2
    # N = 0: nothing launched except clearing the abs-max
    am.fill_(5.0)
    F.ffn_rmsnorm_fwd(empty_bf16(1, C), empty_f32(1), None, am, inp, None, dev_bf16(d["w_norm"]), 1e-5, 0, C)
    torch.cuda.synchronize()
    assert host_f32(am)[0] == 0.0


def test_rmsnorm_zero_rows(F):
    N, C = 8, 512
    say("rmsnorm zero rows")
    z = np.zeros((N, C), np.uint16)
    w = W.uniform_bf16((C,), 0.5, 1.5, 1, 3)
    y, rstd, am = empty_bf16(N, C), empty_f32(N), empty_f32(1)
    F.ffn_rmsnorm_fwd(y, rstd, None, am, dev_bf16(z), None, dev_bf16(w), 1e-5, N, C)
    torch.cuda.synchronize()
    assert np.all(K.bf16_bits_to_f64(host_bits(y)) == 0)
    assert np.allclose(host_f32(rstd), 1 / np.sqrt(np.float32(1e-5)), rtol=1e-6)
    assert host_f32(am)[0] == 0.0


# ----------------------------------------------------------------------------- quantisation

@pytest.mark.parametrize("n,outl", [(64 * 256, False), (300 * 4096, True), (1_000_003, False), (7, False)])
def test_quant_absmax_bit_exact(F, n, outl):
    say(f"quant n={n}")
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32)
    if outl:
        x[rng.random(n) < 1e-3] *= 50
    xb = W.to_bf16_bits(x)
    q, scale, am = empty_u8(n), empty_f32(1), empty_f32(1)
    F.ffn_quant_absmax(q, scale, am, dev_bf16(xb), n, 1)
    torch.cuda.synchronize()
    q_ref, s_ref, am_ref = O.quant_absmax(xb)
    assert host_f32(am)[0] == am_ref
    assert host_f32(scale)[0] == s_ref
    assert np.array_equal(host_u8(q), q_ref)


def _same_codes(got, want, fmt):
    """Codes equal bit for bit, except that a NaN input may come out as any NaN
    code of the format (the sign of a NaN is not specified)."""
    if fmt == "e4m3":
        nan_w, nan_g = (want & 0x7F) == 0x7F, (got & 0x7F) == 0x7F
    else:
        nan_w, nan_g = (want & 0x7F) > 0x7C, (got & 0x7F) > 0x7C
    return np.array_equal(nan_w, nan_g) and np.array_equal(got[~nan_w], want[~nan_w])


def test_quant_every_bf16_pattern_bit_exact(F):
    # all 65536 bf16 patterns (NaN and +-inf included), quantised against
    # several given abs-maxes: a NaN stays NaN, +-inf saturates to +-448
    say("quant exhaustive bf16 patterns")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    n = bits.size
    x = dev_bf16(bits)
    for am_v in [1.0, 3.5, 448.0, 1e-3, 2.0 ** -100, 3.0e38, 0.0]:
        q, scale, am = empty_u8(n), empty_f32(1), dev_f32([am_v])
        F.ffn_quant_absmax(q, scale, am, x, n, 0)
        torch.cuda.synchronize()
        q_ref, s_ref, _ = O.quant_absmax(bits, np.float32(am_v))
        assert host_f32(scale)[0] == s_ref, am_v
        assert _same_codes(host_u8(q), q_ref, "e4m3"), am_v


def test_quant_transpose_every_bf16_pattern_e5m2(F):
    # the e5m2 gradient codes of all 65536 bf16 patterns (NaN and +-inf
    # included), through the quantising transpose, against the oracle
    say("quant transpose e5m2 exhaustive bf16 patterns")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    x = dev_bf16(bits)
    for am_v in [1.0, 57344.0, 3.0e38, 2.0 ** -20]:
        qt, q, sc = empty_u8(256, 256), empty_u8(256, 256), empty_f32(1)
        F.ffn_quant_transpose(qt, q, sc, x, dev_f32([am_v]), 256, 256, 256, code_dtype=F.FFN_E5M2)
        torch.cuda.synchronize()
        q_ref, s_ref, _ = O.quant_absmax(bits, np.float32(am_v), fmt="e5m2")
        assert host_f32(sc)[0] == s_ref, am_v
        assert _same_codes(host_u8(q), q_ref, "e5m2"), am_v
        assert _same_codes(host_u8(qt), q_ref.T, "e5m2"), am_v


def test_absmax_propagates_nan_and_inf(F):
    # max |x| is the unsigned maximum of the bit patterns of |x|: a NaN anywhere
    # makes the abs-max NaN, so the scale and every code are NaN; an infinity
    # gives an infinite abs-max, scale inf and inverse 0 (codes 0, the infinite
    # element NaN).  The same in the RMSNorm and SwiGLU producers.
    say("abs-max with NaN and inf")
    n = 4096 + 37
    base = W.normal_bf16((n,), 1.0, 5, 1)
    for bad, where in ((0x7FC1, 1234), (0xFFC0, 4100), (0x7F80, 99), (0xFF80, 7)):
        b = base.copy()
        b[where] = bad
        q, sc, am = empty_u8(n), empty_f32(1), empty_f32(1)
        F.ffn_quant_absmax(q, sc, am, dev_bf16(b), n, 1)
        torch.cuda.synchronize()
        q_ref, s_ref, am_ref = O.quant_absmax(b)
        g_am = host_f32(am)[0]
        assert (np.isnan(g_am) and np.isnan(am_ref)) or g_am == am_ref, hex(bad)
        assert (np.isnan(host_f32(sc)[0]) and np.isnan(s_ref)) or host_f32(sc)[0] == s_ref, hex(bad)
        assert _same_codes(host_u8(q), q_ref, "e4m3"), hex(bad)
    # producers: a NaN in one row of the RMSNorm input, and in the SwiGLU input
    N, C = 6, 512
    inp = W.normal_bf16((N, C), 1.0, 6, 1)
    inp[3, 17] = 0x7FC0
    y, rstd, am = empty_bf16(N, C), empty_f32(N), empty_f32(1)
    F.ffn_rmsnorm_fwd(y, rstd, None, am, dev_bf16(inp), None, dev_bf16(W.uniform_bf16((C,), 0.5, 1.5, 6, 3)),
                      1e-5, N, C)
    gu = W.normal_bf16((N, 2 * C), 1.0, 6, 2)
    gu[2, 5] = 0x7FC0
    h, amh = empty_bf16(N, C), empty_f32(1)
    F.ffn_swiglu(h, amh, dev_bf16(gu), N, C)
    torch.cuda.synchronize()
    assert np.isnan(host_f32(am)[0]) and np.isnan(host_f32(amh)[0])
    assert np.isnan(host_f32(rstd)[3]) and np.all(np.isfinite(host_f32(rstd)[[0, 1, 2, 4, 5]]))


@pytest.mark.parametrize("rows,cols", [(300, 1024), (64, 4104), (1, 8)])
def test_quant_rows_bit_exact(F, rows, cols):
    say(f"quant_rows {rows}x{cols}")
    w = W.normal_bf16((rows, cols), 0.02, rows + cols, 1)
    q, s = empty_u8(rows, cols), empty_f32(rows)
    F.ffn_quant_rows(q, s, dev_bf16(w), rows, cols)
    torch.cuda.synchronize()
    q_ref, s_ref = O.quant_rows(w)
    assert np.array_equal(host_f32(s), s_ref)
    assert np.array_equal(host_u8(q), q_ref)


# ----------------------------------------------------------------------------- SwiGLU

@pytest.mark.parametrize("N,H", [(64, 768), (33, 14336), (5, 8)])
def test_swiglu(F, N, H):
    say(f"swiglu N={N} H={H}")
    gu = W.normal_bf16((N, 2 * H), 2.0, N + H, 2)
    h, am = empty_bf16(N, H), empty_f32(1)
    F.ffn_swiglu(h, am, dev_bf16(gu), N, H)
    torch.cuda.synchronize()
    h_ref, am_ref = O.swiglu(gu)
    gh = host_bits(h)
    assert ulp_diff(gh, h_ref).max() <= 1           # hardware exp / reciprocal: <= 1 bf16 ulp
    assert np.mean(ulp_diff(gh, h_ref) != 0) < 1e-2
    assert host_f32(am)[0] == np.max(np.abs(K.bf16_bits_to_f64(gh)))


# ----------------------------------------------------------------------------- GEMMs

def _int_bf16(shape, seed, lo=-3, hi=4):
    return W.to_bf16_bits(np.random.default_rng(seed).integers(lo, hi, shape).astype(np.float32))


def _int_e4m3(shape, seed):
    # codes of the integers -4..4 (exact in e4m3): every partial sum is an exact integer
    vals = np.random.default_rng(seed).integers(-4, 5, shape).astype(np.float32)
    return K.e4m3_encode(vals)


GEMM_SHAPES = [(64, 256, 768), (300, 512, 384), (257, 384, 256), (1, 128, 128)]


@pytest.mark.parametrize("N,C,H", GEMM_SHAPES)
def test_gateup_bf16_integer_inputs_bit_exact(F, N, C, H):
    say(f"gateup bf16 int N={N} C={C} H={H}")
    x = _int_bf16((N, C), 1)
    w = _int_bf16((2 * H, C), 2)
    out = empty_bf16(N, 2 * H)
    F.ffn_gateup(out, None, dev_bf16(x), None, dev_bf16(w), None, F.FFN_BF16, 0, N, C, H)
    torch.cuda.synchronize()
    # every partial sum is an integer below 2^24, exact in fp32 in any order;
    # the one bf16 rounding of that exact sum is unique
    assert np.array_equal(host_bits(out), O.gemm_bf16(x, w))


@pytest.mark.parametrize("N,C,H", GEMM_SHAPES)
def test_gateup_fp8_integer_inputs_bit_exact(F, N, C, H):
    say(f"gateup fp8 int N={N} C={C} H={H}")
    qx = _int_e4m3((N, C), 3)
    qw = _int_e4m3((2 * H, C), 4)
    one = dev_f32([1.0])
    out = empty_bf16(N, 2 * H)
    F.ffn_gateup(out, None, dev_u8(qx), one, dev_u8(qw), one, F.FFN_E4M3, 0, N, C, H)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), O.gemm_fp8(qx, np.float32(1), qw, np.float32(1)))


@pytest.mark.parametrize("N,Kd,O", [(257, 4096, 512), (64, 3584, 768)])
def test_same_e4m3_operands_through_both_mfma_paths(F, N, Kd, O):
    """The GEMM bound used for FP8 products: the same e4m3 operands, once as
    bf16 values through the bf16 MFMA path and once as codes through the
    f8f6f4 MFMA path (unit scales), against the exact sum.  (a) Operands whose
    every partial sum is exact in fp32 (values (1 + m/8) 2^e, e in {-1, 0}:
    products are multiples of 2^-8 below 4, sums below 2^14 for K <= 4096):
    the bf16 path gives the exact sum's one bf16 rounding bit for bit.
    (b) Codes of N(0, 1) data (full exponent range): the bf16 path is the
    exact sum rounded once except where fp32 accumulation lands near a bf16
    rounding boundary; the f8f6f4 path stays within
    2^-8 |exact| + 2^-14 sum |a b| everywhere, and differs from the bf16 path
    on a small fraction of outputs."""
    say(f"e4m3 operands through bf16 and f8f6f4 MFMA N={N} K={Kd} O={O}")
    rng = np.random.default_rng(N + Kd + O)
    one = dev_f32([1.0])

    def run(qx, qw):
        xb = W.to_bf16_bits(K.e4m3_decode(qx).astype(np.float32))   # exact: e4m3 values are bf16 values
        wb = W.to_bf16_bits(K.e4m3_decode(qw).astype(np.float32))
        o_b, o_8 = empty_bf16(N, O), empty_bf16(N, O)
        F.ffn_gateup(o_b, None, dev_bf16(xb), None, dev_bf16(wb), None, F.FFN_BF16, 0, N, Kd, O // 2)
        F.ffn_gateup(o_8, None, dev_u8(qx), one, dev_u8(qw), one, F.FFN_E4M3, 0, N, Kd, O // 2)
        torch.cuda.synchronize()
        exact, mag = _exact_and_mag(K.e4m3_decode(qx), K.e4m3_decode(qw))
        return host_bits(o_b), host_bits(o_8), exact, mag

    def narrow(shape):   # sign, e in {-1, 0}, m in 0..7, or zero
        e = rng.integers(6, 8, shape)
        m = rng.integers(0, 8, shape)
        code = (e << 3) | m
        code = np.where(rng.random(shape) < 0.1, 0, code) | (rng.integers(0, 2, shape) << 7)
        return code.astype(np.uint8)
    gb, g8, exact, mag = run(narrow((N, Kd)), narrow((O, Kd)))
    ref = K.f64_to_bf16_bits(exact)
    assert np.array_equal(gb, ref)
    assert np.all(within_dot_bound(g8, exact, mag))
    qx = K.e4m3_encode(rng.standard_normal((N, Kd)).astype(np.float32) * 8)
    qw = K.e4m3_encode(rng.standard_normal((O, Kd)).astype(np.float32) * 8)
    gb, g8, exact, mag = run(qx, qw)
    ref = K.f64_to_bf16_bits(exact)
    assert np.mean(gb != ref) < 1e-3 and ulp_diff(gb, ref).max() <= 1
    assert np.all(within_dot_bound(gb, exact, mag))
    assert np.all(within_dot_bound(g8, exact, mag))
    frac = float(np.mean(g8 != gb))
    say(f"f8f6f4 path differs from the bf16 path on {frac:.2%} of outputs")
    assert frac < 0.05


@pytest.mark.parametrize("fp8", [False, True])
# (256, 4096, 1792): the gate+up shape of one GPU's share under 8-way tensor parallelism
@pytest.mark.parametrize("N,C,H", [(64, 256, 768), (300, 512, 384), (1100, 256, 7680), (256, 4096, 1792)])
def test_gateup_random_and_fused_equals_unfused(F, fp8, N, C, H):
    say(f"gateup random fp8={fp8} N={N} C={C} H={H}")
    d = W.block_inputs(N, C, H, seed=N + C + H, w_std=0.0)
    if fp8:
        qx, sx, _ = O.quant_absmax(d["inp"])
        qw, sw, _ = O.quant_absmax(d["w_gu"])
        xa, wa, xs, ws, dt = dev_u8(qx), dev_u8(qw), dev_f32([sx]), dev_f32([sw]), F.FFN_E4M3
        ref = O.gemm_fp8(qx, sx, qw, sw)
        exact, mag = _exact_and_mag(K.e4m3_decode(qx), K.e4m3_decode(qw), float(np.float32(sx * sw)))
    else:
        xa, wa, xs, ws, dt = dev_bf16(d["inp"]), dev_bf16(d["w_gu"]), None, None, F.FFN_BF16
        ref = O.gemm_bf16(d["inp"], d["w_gu"])
        exact, mag = _exact_and_mag(K.bf16_bits_to_f64(d["inp"]), K.bf16_bits_to_f64(d["w_gu"]))
    gu = empty_bf16(N, 2 * H)
    F.ffn_gateup(gu, None, xa, xs, wa, ws, dt, 0, N, C, H)
    h_f, am_f = empty_bf16(N, H), empty_f32(1)
    F.ffn_gateup(h_f, am_f, xa, xs, wa, ws, dt, 1, N, C, H)
    h_u, am_u = empty_bf16(N, H), empty_f32(1)
    F.ffn_swiglu(h_u, am_u, gu, N, H)
    torch.cuda.synchronize()
    g_gu = host_bits(gu)
    assert rel_err(g_gu, ref) < 1e-2
    assert np.all(within_dot_bound(g_gu, exact, mag))
    # the fused epilogue is the unfused pair exactly
    assert np.array_equal(host_bits(h_f), host_bits(h_u))
    assert host_f32(am_f)[0] == host_f32(am_u)[0]
    h_ref, _ = O.swiglu(ref)
    assert rel_err(host_bits(h_f), h_ref) < 3e-2


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("N,C,H", [(64, 256, 768), (300, 512, 384), (1100, 256, 7680)])
def test_gateup_swiglu_quant_known_absmax(F, fp8, N, C, H):
    # the one-pass form equals the two-pass chain (fused gate+up -> bf16 h ->
    # ffn_quant_absmax with the abs-max given) bit for bit, and the oracle's
    # quantiser on the same h, for the exact abs-max, a stale smaller one
    # (saturating codes) and zero
    say(f"gateup swiglu quant fp8={fp8} N={N} C={C} H={H}")
    d = W.block_inputs(N, C, H, seed=N + C + H + 7, w_std=0.0)
    if fp8:
        qx, sx, _ = O.quant_absmax(d["inp"])
        qw, sw, _ = O.quant_absmax(d["w_gu"])
        xa, wa, xs, ws, dt = dev_u8(qx), dev_u8(qw), dev_f32([sx]), dev_f32([sw]), F.FFN_E4M3
    else:
        xa, wa, xs, ws, dt = dev_bf16(d["inp"]), dev_bf16(d["w_gu"]), None, None, F.FFN_BF16
    h, am = empty_bf16(N, H), empty_f32(1)
    F.ffn_gateup(h, am, xa, xs, wa, ws, dt, 1, N, C, H)
    torch.cuda.synchronize()
    amax = float(host_f32(am)[0])
    hb = host_bits(h)
    for known in (amax, amax * 0.5, 0.0):
        q2, s2 = empty_u8(N, H), empty_f32(1)
        F.ffn_quant_absmax(q2, s2, dev_f32([known]), h, N * H, 0)
        q, qs, ham = empty_u8(N, H), empty_f32(1), empty_f32(1)
        F.ffn_gateup_swiglu_quant(q, qs, ham, dev_f32([known]), xa, xs, wa, ws, dt, N, C, H)
        torch.cuda.synchronize()
        assert torch.equal(q, q2)
        assert host_f32(qs)[0] == host_f32(s2)[0]
        assert host_f32(ham)[0] == np.float32(amax)
        qo, so, _ = O.quant_absmax(hb, np.float32(known))
        assert np.array_equal(host_u8(q), qo)
        assert host_f32(qs)[0] == so


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("N,H,C", [(64, 768, 256), (300, 384, 512), (513, 256, 384), (3100, 384, 5248),
                                   (256, 1792, 4096)])
def test_down(F, fp8, N, H, C):
    say(f"down fp8={fp8} N={N} H={H} C={C}")
    h = W.normal_bf16((N, H), 1.0, N + H, 3)
    w = W.normal_bf16((C, H), 1 / np.sqrt(H), N + H, 4)
    if fp8:
        qh, sh, _ = O.quant_absmax(h)
        qw, sw, _ = O.quant_absmax(w)
        args = (dev_u8(qh), dev_f32([sh]), dev_u8(qw), dev_f32([sw]), F.FFN_E4M3)
        ref = O.gemm_fp8(qh, sh, qw, sw)
        exact, mag = _exact_and_mag(K.e4m3_decode(qh), K.e4m3_decode(qw), float(np.float32(sh * sw)))
    else:
        args = (dev_bf16(h), None, dev_bf16(w), None, F.FFN_BF16)
        ref = O.gemm_bf16(h, w)
        exact, mag = _exact_and_mag(K.bf16_bits_to_f64(h), K.bf16_bits_to_f64(w))
    out = empty_bf16(N, C)
    F.ffn_down(out, *args, N, H, C)
    torch.cuda.synchronize()
    g = host_bits(out)
    assert rel_err(g, ref) < 1e-2
    assert np.all(within_dot_bound(g, exact, mag))
    if not fp8:  # fp32 accumulation: beyond the last bit only where the sum cancels
        assert np.mean(ulp_diff(g, ref) > 1) < 1e-3


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_gemm_writes_stay_inside_the_output(F, fp8, fused):
    # More tiles than workgroups (each workgroup walks several), a ragged last
    # token tile and, for the down projection, a half-filled last feature
    # tile: nothing past the output may be written.
    if fused:
        N, R, O_ = 1100, 384, 7680          # gate+up, H = 7680: 60 x 5 tiles
    else:
        N, R, O_ = 3100, 384, 5248          # down, C = 41 * 128: 21 x 13 tiles
    say(f"gemm guard fp8={fp8} fused={fused}")
    x = _int_e4m3((N, R), 11) if fp8 else _int_bf16((N, R), 11)
    w_rows = 2 * O_ if fused else O_
    w = _int_e4m3((w_rows, R), 12) if fp8 else _int_bf16((w_rows, R), 12)
    guard = torch.full(((N + 3) * O_,), 0x7B7B, dtype=torch.int16, device="cuda")
    out = guard[: N * O_].view(N, O_).view(torch.bfloat16)
    one = dev_f32([1.0])
    xa, wa = (dev_u8(x), dev_u8(w)) if fp8 else (dev_bf16(x), dev_bf16(w))
    xs, ws, dt = (one, one, F.FFN_E4M3) if fp8 else (None, None, F.FFN_BF16)
    if fused:
        F.ffn_gateup(out, None, xa, xs, wa, ws, dt, 1, N, R, O_)
    else:
        F.ffn_down(out, xa, xs, wa, ws, dt, N, R, O_)
    torch.cuda.synchronize()
    assert torch.all(guard[N * O_:] == 0x7B7B)
    ref = O.gemm_fp8(x, np.float32(1), w, np.float32(1)) if fp8 else O.gemm_bf16(x, w)
    g = host_bits(out)
    if fused:
        # integer g and u are exact; only the hardware exp / reciprocal of the
        # SiLU can move a result by one bf16 step, or, where silu(g) underflows
        # (g below about -80), leave 0 for a value under 1e-30
        h_ref, _ = O.swiglu(ref)
        tiny = (np.abs(K.bf16_bits_to_f64(h_ref)) < 1e-30) & (np.abs(K.bf16_bits_to_f64(g)) < 1e-30)
        assert np.all((ulp_diff(g, h_ref) <= 1) | tiny)
    else:
        assert np.array_equal(g, ref)


def test_gemm_integer_down_bit_exact_and_deterministic(F):
    N, H, C = 260, 512, 384
    say("down int bit-exact")
    h = _int_bf16((N, H), 5)
    w = _int_bf16((C, H), 6)
    out1, out2 = empty_bf16(N, C), empty_bf16(N, C)
    F.ffn_down(out1, dev_bf16(h), None, dev_bf16(w), None, F.FFN_BF16, N, H, C)
    F.ffn_down(out2, dev_bf16(h), None, dev_bf16(w), None, F.FFN_BF16, N, H, C)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out1), O.gemm_bf16(h, w))
    assert torch.equal(out1, out2)


def test_zero_rows_still_write_the_per_tensor_outputs(F):
    # N = 0: no rows are written; an abs-max of no elements is 0 (the _acc form
    # leaves its word as found) and the quantising calls still write their
    # scale from the given abs-max (the oracle's scale of that abs-max)
    say("zero rows: GEMM entry points and the quantising transpose")
    C, H = 256, 256
    xs, ws = dev_f32([0.5]), dev_f32([0.25])
    x, w, wd = empty_u8(1, C).zero_(), empty_u8(2 * H, C).zero_(), empty_u8(C, H).zero_()
    h = empty_bf16(1, H).fill_(3.0)
    am = dev_f32([7.0])
    F.ffn_gateup(h, am, x, xs, w, ws, F.FFN_E4M3, 1, 0, C, H)
    acc = dev_f32([7.0])
    F.ffn_gateup_acc(h, acc, x, xs, w, ws, F.FFN_E4M3, 0, C, H)
    q, qs, ham = empty_u8(1, H).fill_(0x11), dev_f32([-1.0]), dev_f32([7.0])
    F.ffn_gateup_swiglu_quant(q, qs, ham, dev_f32([3.5]), x, xs, w, ws, F.FFN_E4M3, 0, C, H)
    qs0 = dev_f32([-1.0])
    F.ffn_gateup_swiglu_quant(q, qs0, None, dev_f32([0.0]), x, xs, w, ws, F.FFN_E4M3, 0, C, H)
    out = empty_bf16(1, C).fill_(2.0)
    F.ffn_down(out, empty_u8(1, H).zero_(), xs, wd, ws, F.FFN_E4M3, 0, H, C)
    xb = empty_bf16(16, 16).zero_()
    sc4, sc5 = dev_f32([-1.0]), dev_f32([-1.0])
    F.ffn_quant_transpose(empty_u8(16, 16), None, sc4, xb, dev_f32([114.0]), 16, 0, 16)
    F.ffn_quant_transpose(empty_u8(16, 16), None, sc5, xb, dev_f32([114.0]), 16, 0, 16, code_dtype=F.FFN_E5M2)
    torch.cuda.synchronize()
    assert host_f32(am)[0] == 0.0 and host_f32(acc)[0] == 7.0 and host_f32(ham)[0] == 0.0
    assert host_f32(qs)[0] == O.quant_absmax(np.zeros(1, np.uint16), np.float32(3.5))[1]
    assert host_f32(qs0)[0] == 1.0
    assert host_f32(sc4)[0] == O.quant_absmax(np.zeros(1, np.uint16), np.float32(114.0))[1]
    assert host_f32(sc5)[0] == O.quant_absmax(np.zeros(1, np.uint16), np.float32(114.0), fmt="e5m2")[1]
    assert np.all(host_u8(q) == 0x11) and torch.all(h == 3.0) and torch.all(out == 2.0)


# ----------------------------------------------------------------------------- decode

# (1, 4096, 1792): one GPU's share of the single-token decode under 8-way tensor parallelism
@pytest.mark.parametrize("M,C,H", [(1, 256, 768), (1, 4096, 1024), (1, 3584, 384), (2, 1152, 640), (3, 512, 640), (4, 1024, 9216), (4, 640, 2304), (16, 384, 896),
                                   (32, 256, 256), (1, 4096, 1792)])
def test_decode(F, M, C, H):
    say(f"decode M={M} C={C} H={H}")
    d = W.decode_inputs(M, C, H, seed=M * 13 + C + H)
    wq, ws = {}, {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        q, s = empty_u8(rows, cols), empty_f32(rows)
        F.ffn_quant_rows(q, s, dev_bf16(d[k]), rows, cols)
        wq[k], ws[k] = q, s
    out, h = empty_bf16(M, C), empty_bf16(M, H)
    xd = dev_bf16(d["x"])
    F.ffn_decode_gemv(out, h, xd, wq["w_gate"], ws["w_gate"], wq["w_up"], ws["w_up"],
                      wq["w_down"], ws["w_down"], M, C, H)
    # the pre-bound form issues the identical call
    out2, h2 = empty_bf16(M, C), empty_bf16(M, H)
    call = F.bind_decode_gemv(out2, h2, xd, wq["w_gate"], ws["w_gate"], wq["w_up"], ws["w_up"],
                              wq["w_down"], ws["w_down"], M, C, H)
    call()
    call()
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(h2, h)
    ref_q = {k: O.quant_rows(d[k]) for k in ("w_gate", "w_up", "w_down")}
    for k in ref_q:
        assert np.array_equal(host_u8(wq[k]), ref_q[k][0])
        assert np.array_equal(host_f32(ws[k]), ref_q[k][1])
    (qg, sg), (qu, su), (qd, sd) = ref_q["w_gate"], ref_q["w_up"], ref_q["w_down"]
    y_ref, h_ref = O.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    gh, gy = host_bits(h), host_bits(out)
    assert rel_err(gh, h_ref) < 2e-2
    # the down GEMV given the GPU's own h
    assert rel_err(gy, O.decode_down(gh, qd, sd)) < 1e-2
    assert rel_err(gy, y_ref) < 3e-2


def _decode_weights(F, d):
    wq, ws = {}, {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        q, s = empty_u8(rows, cols), empty_f32(rows)
        F.ffn_quant_rows(q, s, dev_bf16(d[k]), rows, cols)
        wq[k], ws[k] = q, s
    return wq, ws


# partial windows of 1024 (FP8) and 512 (bf16) weights per row in C and in H
ARM_SHAPES = [(1, 256, 768), (1, 3584, 384), (2, 1152, 640), (3, 512, 640), (4, 640, 2304), (4, 4096, 1024)]


@pytest.mark.parametrize("M,C,H", ARM_SHAPES)
def test_decode_arms_agree_bit_for_bit(F, M, C, H):
    say(f"decode arms M={M} C={C} H={H}")
    d = W.decode_inputs(M, C, H, seed=M * 31 + C + H)
    wq, ws = _decode_weights(F, d)
    xd = dev_bf16(d["x"])
    args = (xd, wq["w_gate"], ws["w_gate"], wq["w_up"], ws["w_up"], wq["w_down"], ws["w_down"])
    out, h = empty_bf16(M, C), empty_bf16(M, H)
    F.ffn_decode_gemv(out, h, *args, M, C, H)
    res = {}
    for arm in (F.FFN_DECODE_SPLIT_SILU, F.FFN_DECODE_SILU_INPUT, F.FFN_DECODE_PER_PROJECTION):
        o2, h2, gu = empty_bf16(M, C).fill_(7.0), empty_bf16(M, H).fill_(7.0), empty_bf16(M, 2 * H).fill_(7.0)
        F.ffn_decode_gemv_arm(o2, h2, gu, *args, arm, M, C, H)
        res[arm] = (o2, h2, gu)
    torch.cuda.synchronize()
    for arm, (o2, h2, gu) in res.items():
        assert torch.equal(o2, out), arm
        if arm != F.FFN_DECODE_SILU_INPUT:
            assert torch.equal(h2, h), arm
        if arm != F.FFN_DECODE_SPLIT_SILU:
            # the workspace holds g then u: the oracle's SwiGLU of it is the split
            # arm's h up to the hardware exp's last bit
            dh = ulp_diff(O.swiglu(host_bits(gu))[0], host_bits(h))
            assert dh.max() <= 1 and np.mean(dh != 0) < 1e-2, arm
    # and the split arm against the oracle, as in test_decode
    ref_q = {k: O.quant_rows(d[k]) for k in ("w_gate", "w_up", "w_down")}
    (qg, sg), (qu, su), (qd, sd) = ref_q["w_gate"], ref_q["w_up"], ref_q["w_down"]
    y_ref, h_ref = O.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    assert rel_err(host_bits(h), h_ref) < 2e-2
    assert rel_err(host_bits(out), y_ref) < 3e-2


@pytest.mark.parametrize("M,C,H", ARM_SHAPES + [(1, 128, 128)])
def test_decode_bf16_weights(F, M, C, H):
    say(f"decode bf16 weights M={M} C={C} H={H}")
    d = W.decode_inputs(M, C, H, seed=M * 17 + C + H)
    out, h = empty_bf16(M, C).fill_(7.0), empty_bf16(M, H).fill_(7.0)
    F.ffn_decode_gemv_bf16(out, h, dev_bf16(d["x"]), dev_bf16(d["w_gate"]), dev_bf16(d["w_up"]),
                           dev_bf16(d["w_down"]), M, C, H)
    torch.cuda.synchronize()
    y_ref, h_ref = O.decode_gemv_bf16(d["x"], d["w_gate"], d["w_up"], d["w_down"])
    gh, gy = host_bits(h), host_bits(out)
    # fp32 sums in another order than the oracle's fp64: g and u can land one
    # bf16 ulp apart, rarely
    assert rel_err(gh, h_ref) < 2e-2
    # the down GEMV given the GPU's own h: one rounding of an fp32 sum
    y_cond = O.gemm_bf16(gh, d["w_down"])
    assert ulp_diff(gy, y_cond).max() <= 1
    assert rel_err(gy, y_ref) < 2e-2


@pytest.mark.parametrize("rows,cols", [(16, 128), (48, 384), (384, 1152)])
def test_decode_pack_weight_layout(F, rows, cols):
    """The packed layout is the re-indexing the header defines: piece p = row
    16 rb + l % 16, codes 64 kc + 16 (l / 16) .. + 15, l = p % 64,
    p / 64 = kc * rows / 16 + rb."""
    say(f"decode pack rows={rows} cols={cols}")
    w = np.random.default_rng(rows + cols).integers(0, 256, (rows, cols)).astype(np.uint8)
    out = empty_u8(rows, cols).fill_(0)
    F.ffn_decode_pack_weight(out, dev_u8(w), rows, cols)
    torch.cuda.synchronize()
    want = w.reshape(rows // 16, 16, cols // 64, 4, 16).transpose(2, 0, 3, 1, 4).reshape(rows, cols)
    assert np.array_equal(host_u8(out).reshape(rows, cols), want)


# Up to 14 tokens the dual pass loads the activations with every item's
# weights (at any C: (3, 4224, 256) is past the LDS copy's limit); from 15 to
# 16 tokens with C <= 4096 it keeps them in LDS (a half last chunk at C = 640;
# C = 4096 fills the LDS copy), above C = 4096 it reads them from the
# fragment-order copy in the workspace.  Up to
# 16 tokens the down pass is split along K over workgroups (slices of one
# 64-code piece at H = 128 x 1 group of rows, up to 64 pieces) whose fp32
# partial sums a second kernel adds in slice order; 17 to 32 tokens take two
# token blocks.  (16, 3584, 4736) is one GPU's share of the Qwen2-7B-shaped
# decode under 4-way tensor parallelism.
PACKED_SHAPES = [(1, 1152, 640), (5, 3584, 384), (16, 384, 896), (16, 3584, 18944), (3, 4224, 256), (17, 256, 640),
                 (32, 256, 256), (1, 1152, 4096), (5, 4096, 4096), (16, 384, 8192), (13, 640, 4096),
                 (16, 4096, 14336), (2, 128, 128), (9, 128, 8192), (16, 8192, 256), (16, 3584, 4736),
                 (14, 640, 1024), (15, 640, 1024)]


@pytest.mark.parametrize("M,C,H", PACKED_SHAPES)
def test_decode_packed(F, M, C, H):
    """ffn_decode_gemv_packed on packed weights against the oracle, as
    test_decode; the bound form repeats the call exactly.  (16, 3584, 18944)
    is the 16-token decode of the Qwen2-7B-shaped step."""
    say(f"decode packed M={M} C={C} H={H}")
    d = W.decode_inputs(M, C, H, seed=M * 19 + C + H)
    wq, ws = _decode_weights(F, d)
    pk = {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        pk[k] = empty_u8(rows, cols)
        F.ffn_decode_pack_weight(pk[k], wq[k], rows, cols)
    wsp = empty_bf16(F.ffn_decode_packed_workspace_bytes(M, C, H) // 2).fill_(5.0)
    out, h = empty_bf16(M, C).fill_(7.0), empty_bf16(M, H).fill_(7.0)
    xd = dev_bf16(d["x"])
    args = (xd, pk["w_gate"], ws["w_gate"], pk["w_up"], ws["w_up"], pk["w_down"], ws["w_down"], M, C, H)
    F.ffn_decode_gemv_packed(out, h, wsp, *args)
    out2, h2 = empty_bf16(M, C), empty_bf16(M, H)
    call = F.bind_decode_gemv_packed(out2, h2, wsp, *args)
    call()
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(h2, h)
    ref_q = {k: O.quant_rows(d[k]) for k in ("w_gate", "w_up", "w_down")}
    (qg, sg), (qu, su), (qd, sd) = ref_q["w_gate"], ref_q["w_up"], ref_q["w_down"]
    y_ref, h_ref = O.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    gh, gy = host_bits(h), host_bits(out)
    assert rel_err(gh, h_ref) < 2e-2
    assert rel_err(gy, O.decode_down(gh, qd, sd)) < 1e-2
    assert rel_err(gy, y_ref) < 3e-2


def _bf16_ulp(v):
    """Spacing of bf16 values at |v| (8 significant bits; zero and
    subnormals take the smallest normal spacing)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _assert_h_differs_by_sum_order_only(h_a, h_b, x_bits, qg, sg, qu, su):
    """Two decode forms that take the same products in another fp32 order:
    g and u may move by the order's error (at most 2^-15 of the row's sum of
    magnitudes over the fp32 partial sums of these K; both orders' errors
    together) plus one bf16 ulp where their rounding flips, and h by what
    that moves silu(g) u (first order, with a factor of 2 for the second
    order terms) plus one ulp of its own rounding.  Cancellation in g or u
    (a sum far smaller than its terms), or a steep silu at a negative g, lets
    h move many ulps, so the bound is taken element by element from fp64
    values of g and u."""
    xf = O.bf16_bits_to_f64(x_bits)
    wg = O.e4m3_decode(host_u8(qg)) * host_f32(sg).astype(np.float64)[:, None]
    wu = O.e4m3_decode(host_u8(qu)) * host_f32(su).astype(np.float64)[:, None]
    g, u = xf @ wg.T, xf @ wu.T
    mg, mu = np.abs(xf) @ np.abs(wg).T, np.abs(xf) @ np.abs(wu).T
    sig = 1.0 / (1.0 + np.exp(-g))
    eps = 2.0 ** -15
    move = (np.abs(u * (sig + g * sig * (1.0 - sig))) * (_bf16_ulp(g) + eps * mg)
            + np.abs(g * sig) * (_bf16_ulp(u) + eps * mu))
    href = g * sig * u
    bound = 2.0 * move + _bf16_ulp(href)
    ha, hb = O.bf16_bits_to_f64(h_a), O.bf16_bits_to_f64(h_b)
    dh = ulp_diff(h_a, h_b)
    say(f"  h: {np.mean(dh != 0):.4f} of the elements differ, {np.mean(dh > 2):.5f} by more than 2 ulps, "
        f"max {dh.max()} ulps; max |diff| / bound {np.max(np.abs(ha - hb) / bound):.3f}")
    assert np.all(np.abs(ha - hb) <= bound)
    assert np.mean(dh != 0) < 5e-2


def test_decode_packed_one_and_two_token_blocks_agree(F):
    """The 16-token form (activations in LDS, down pass split along K) and the
    two-token-block form (the same 16 tokens plus one) on the same rows: the
    sums differ only in fp32 order, so h differs by what that order moves
    (cancelling sums aside, an ulp or two on a small fraction of the
    elements); y agrees within the down pass's rounding."""
    C, H = 1152, 4096
    say(f"decode packed 16 vs 17 tokens C={C} H={H}")
    d = W.decode_inputs(17, C, H, seed=4242)
    wq, ws = _decode_weights(F, d)
    pk = {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        pk[k] = empty_u8(rows, cols)
        F.ffn_decode_pack_weight(pk[k], wq[k], rows, cols)
    wts = (pk["w_gate"], ws["w_gate"], pk["w_up"], ws["w_up"], pk["w_down"], ws["w_down"])
    x17 = dev_bf16(d["x"])
    res = {}
    for M in (16, 17):
        wsp = empty_bf16(F.ffn_decode_packed_workspace_bytes(M, C, H) // 2)
        o, h = empty_bf16(M, C), empty_bf16(M, H)
        F.ffn_decode_gemv_packed(o, h, wsp, x17[:M].contiguous(), *wts, M, C, H)
        res[M] = (o, h)
    torch.cuda.synchronize()
    _assert_h_differs_by_sum_order_only(host_bits(res[16][1]), host_bits(res[17][1][:16]), d["x"][:16],
                                        wq["w_gate"], ws["w_gate"], wq["w_up"], ws["w_up"])
    assert rel_err(host_bits(res[16][0]), host_bits(res[17][0][:16])) < 1e-2


@pytest.mark.parametrize("C,H", [(3584, 18944), (4096, 1152)])
def test_decode_packed_register_and_lds_forms_agree(F, C, H):
    """Twelve tokens (activations loaded with every item's weights, 2-KiB
    groups) and the same twelve plus one (activations copied into LDS, 8-KiB
    groups): each wave starts its walk at a group that depends on the group
    size, so the sums differ only in fp32 order and h by what that order
    moves; y agrees within the down pass's rounding."""
    say(f"decode packed 12 vs 13 tokens C={C} H={H}")
    d = W.decode_inputs(13, C, H, seed=C + H + 1213)
    wq, ws = _decode_weights(F, d)
    pk = {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        pk[k] = empty_u8(rows, cols)
        F.ffn_decode_pack_weight(pk[k], wq[k], rows, cols)
    wts = (pk["w_gate"], ws["w_gate"], pk["w_up"], ws["w_up"], pk["w_down"], ws["w_down"])
    x13 = dev_bf16(d["x"])
    res = {}
    for M in (12, 13):
        wsp = empty_bf16(F.ffn_decode_packed_workspace_bytes(M, C, H) // 2)
        o, h = empty_bf16(M, C), empty_bf16(M, H)
        F.ffn_decode_gemv_packed(o, h, wsp, x13[:M].contiguous(), *wts, M, C, H)
        res[M] = (o, h)
    torch.cuda.synchronize()
    _assert_h_differs_by_sum_order_only(host_bits(res[12][1]), host_bits(res[13][1][:12]), d["x"][:12],
                                        wq["w_gate"], ws["w_gate"], wq["w_up"], ws["w_up"])
    assert rel_err(host_bits(res[12][0]), host_bits(res[13][0][:12])) < 1e-2


def test_decode_packed_workspace_reuse(F):
    """One workspace, a 32-token call and then a 5-token one: the second
    result equals a call on a fresh workspace bit for bit (nothing of the
    first call's tokens leaks into the second)."""
    say("decode packed workspace reuse")
    C, H = 384, 512
    d = W.decode_inputs(32, C, H, seed=123)
    wq, ws = _decode_weights(F, d)
    pk = {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        pk[k] = empty_u8(rows, cols)
        F.ffn_decode_pack_weight(pk[k], wq[k], rows, cols)
    wts = (pk["w_gate"], ws["w_gate"], pk["w_up"], ws["w_up"], pk["w_down"], ws["w_down"])
    shared = empty_bf16(F.ffn_decode_packed_workspace_bytes(32, C, H) // 2)
    x32 = dev_bf16(d["x"])
    F.ffn_decode_gemv_packed(empty_bf16(32, C), empty_bf16(32, H), shared, x32, *wts, 32, C, H)
    x5 = x32[:5].contiguous()
    o_a, h_a = empty_bf16(5, C), empty_bf16(5, H)
    F.ffn_decode_gemv_packed(o_a, h_a, shared, x5, *wts, 5, C, H)
    fresh = empty_bf16(F.ffn_decode_packed_workspace_bytes(5, C, H) // 2).fill_(-3.0)
    o_b, h_b = empty_bf16(5, C), empty_bf16(5, H)
    F.ffn_decode_gemv_packed(o_b, h_b, fresh, x5, *wts, 5, C, H)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(h_a, h_b)


def test_decode_block_packed(F):
    """DecodeBlockPacked (packed copies of DecodeBlock's codes) against
    DecodeBlock on the same master weights and through set_fp8_weights, and
    against the oracle."""
    from transformer_ffn_block_residual_amd import block
    M, C, H = 12, 512, 1024
    say(f"decode block packed M={M} C={C} H={H}")
    d = W.decode_inputs(M, C, H, seed=321)
    rows = block.DecodeBlock(M, C, H)
    rows.load_master_weights(d["w_gate"], d["w_up"], d["w_down"])
    pk = block.DecodeBlockPacked(M, C, H)
    pk.load_master_weights(d["w_gate"], d["w_up"], d["w_down"])
    pk2 = block.DecodeBlockPacked(M, C, H)
    pk2.set_fp8_weights(rows.wg, rows.sg, rows.wu, rows.su, rows.wd, rows.sd)
    x = dev_bf16(d["x"])
    y_rows = rows.forward(x).clone()
    y_pk = pk.forward(x).clone()
    pk2.bind(x)()
    torch.cuda.synchronize()
    assert torch.equal(pk2.out, y_pk) and torch.equal(pk2.h, pk.h)
    (qg, sg), (qu, su), (qd, sd) = (O.quant_rows(d[k]) for k in ("w_gate", "w_up", "w_down"))
    y_ref, h_ref = O.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    assert rel_err(host_bits(pk.h)[:M], h_ref) < 2e-2
    assert rel_err(host_bits(y_pk)[:M], y_ref) < 3e-2
    assert rel_err(host_bits(y_pk)[:M], host_bits(y_rows)[:M]) < 2e-2
    with pytest.raises(NotImplementedError):
        pk.forward_arm(x, F.FFN_DECODE_SILU_INPUT)


def test_decode_empty_batch(F):
    say("decode M=0")
    C, H = 256, 256
    z = empty_u8(H, C).zero_()
    s = empty_f32(H).fill_(1.0)
    F.ffn_decode_gemv(empty_bf16(1, C), empty_bf16(1, H), empty_bf16(1, C), z, s, z, s, z, s, 0, C, H)
    torch.cuda.synchronize()
