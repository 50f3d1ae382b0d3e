"""Pins for the oracle's FFN steps.

Every check compares the oracle with something it does not call: torch's CPU
routines (``rms_norm``, ``silu``, bf16 addition, float8 conversion, float64
matmul), brute-force loops over exact fractions, closed forms, and invariants
of the block that a dropped term, a swapped gate/up half, a transposed
operand or a wrong scale would break.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle import codecs as K
from transformer_ffn_block_residual_amd import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bits_to_torch(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place (same-sign finite values)."""
    a = np.asarray(a_bits).astype(np.int32)
    b = np.asarray(b_bits).astype(np.int32)
    ka = np.where(a & 0x8000, -(a & 0x7FFF), a)
    kb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ka - kb)


# ----------------------------------------------------------------------------- residual + RMSNorm

def test_residual_add_matches_torch_bf16_add():
    rng = np.random.default_rng(1)
    a = W.to_bf16_bits(rng.standard_normal((64, 512)).astype(np.float32) * 10)
    b = W.to_bf16_bits(rng.standard_normal((64, 512)).astype(np.float32) * 1e-2)
    want = (bits_to_torch(a) + bits_to_torch(b)).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.residual_add(a, b), want)


def test_rmsnorm_matches_torch_rms_norm():
    d = W.block_inputs(37, 384, 128, seed=5)
    r, y, rstd, am = O.rmsnorm_fwd(d["inp"], d["addend"], d["w_norm"], 1e-5)
    rt = bits_to_torch(r).double()
    wt = bits_to_torch(d["w_norm"]).double()
    yt = F.rms_norm(rt, (384,), weight=wt, eps=1e-5)
    y_ref = W.to_bf16_bits(yt.float().numpy())  # fp64 -> fp32 -> bf16 may double-round
    assert ulp_diff(y, y_ref).max() <= 1
    assert np.mean(ulp_diff(y, y_ref) != 0) < 1e-3
    rstd_ref = torch.rsqrt(rt.pow(2).mean(-1) + 1e-5).numpy()
    assert np.max(np.abs(rstd / rstd_ref - 1)) < 2 ** -23
    assert am == np.max(np.abs(K.bf16_bits_to_f64(y)))


def test_rmsnorm_unit_weight_gives_unit_rms():
    rng = np.random.default_rng(2)
    x = W.to_bf16_bits(rng.standard_normal((50, 1024)).astype(np.float32) * rng.uniform(0.01, 100, (50, 1)).astype(np.float32))
    ones = W.to_bf16_bits(np.ones(1024, np.float32))
    eps = 1e-5
    _, y, rstd, _ = O.rmsnorm_fwd(x, None, ones, eps)
    xv = K.bf16_bits_to_f64(x)
    m = np.mean(xv ** 2, axis=1)
    ms_y = np.mean(K.bf16_bits_to_f64(y) ** 2, axis=1)
    # mean(y^2) = m / (m + eps), up to bf16 rounding of each y (rel 2^-8 per element)
    assert np.allclose(ms_y, m / (m + eps), rtol=2 ** -7)


def test_rmsnorm_degenerate_rows():
    C = 256
    w = W.to_bf16_bits(np.linspace(0.5, 1.5, C).astype(np.float32))
    zero = np.zeros((1, C), np.uint16)
    r, y, rstd, am = O.rmsnorm_fwd(zero, zero, w, 1e-5)
    assert np.all(K.bf16_bits_to_f64(y) == 0) and am == 0
    assert rstd[0] == np.float32(1 / np.sqrt(np.float64(np.float32(1e-5))))
    # a constant row c: rstd = 1/sqrt(c^2 + eps), y = c * rstd * w
    c = W.to_bf16_bits(np.full((1, C), 3.0, np.float32))
    _, y, rstd, _ = O.rmsnorm_fwd(c, None, w, 0.0)
    assert rstd[0] == np.float32(1 / 3)
    assert np.array_equal(y, W.to_bf16_bits((3.0 * np.float64(np.float32(1 / 3)) * K.bf16_bits_to_f64(w)).astype(np.float32)[None]))


def test_rmsnorm_hand_worked_row():
    # r = [3, 4, 0, 0] (+ zero addend), eps = 0: mean r^2 = 25/4, rstd = 0.4
    # y = [1.2, 1.6, 0, 0] rounded to bf16: 1.2 -> 1.203125 (0x3F9A), 1.6 -> 1.6015625 (0x3FCD)
    inp = W.to_bf16_bits(np.array([[3, 4, 0, 0]], np.float32))
    zero = np.zeros((1, 4), np.uint16)
    ones = W.to_bf16_bits(np.ones(4, np.float32))
    r, y, rstd, am = O.rmsnorm_fwd(inp, zero, ones, 0.0)
    assert list(r[0]) == list(inp[0])
    assert rstd[0] == np.float32(0.4)
    assert list(y[0]) == [0x3F9A, 0x3FCD, 0, 0]
    assert am == np.float32(1.6015625)


# ----------------------------------------------------------------------------- quantisation

def test_quant_maps_absmax_to_448_and_respects_bounds():
    for seed, outl in [(1, False), (2, True)]:
        d = W.block_inputs(64, 512, 128, seed=seed, outliers=outl)
        x = d["inp"]
        q, scale, am = O.quant_absmax(x)
        xv = K.bf16_bits_to_f64(x)
        assert am == np.float32(np.max(np.abs(xv)))
        assert scale == np.float32(np.float64(am) / 448.0)
        iam = np.argmax(np.abs(xv))
        assert q.reshape(-1)[iam] in (0x7E, 0xFE)
        dq = K.e4m3_decode(q)
        assert np.all(np.abs(dq) <= 448)
        assert np.all(np.isfinite(dq))
        # dequantisation error: half a step of the e4m3 grid around x*inv
        p = np.abs(xv * (448.0 / am))
        step = np.where(p >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(p, 2 ** -6))) - 3), 2.0 ** -9)
        assert np.all(np.abs(np.abs(dq) - p) <= step / 2 * (1 + 1e-6) + 1e-12)
        # sign and monotonicity
        assert np.all((xv > 0) <= (dq >= 0)) and np.all((xv < 0) <= (dq <= 0))
        o = np.argsort(xv.reshape(-1), kind="stable")
        assert np.all(np.diff(dq.reshape(-1)[o]) >= 0)


def test_quant_matches_torch_float8():
    d = W.block_inputs(64, 512, 128, seed=9, outliers=True)
    x = d["addend"]
    q, scale, am = O.quant_absmax(x)
    xt = bits_to_torch(x).float()
    inv = torch.tensor(448.0, dtype=torch.float32) / torch.tensor(float(am), dtype=torch.float32)
    want = torch.clamp(xt * inv, -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)


def test_quant_zero_tensor_and_given_absmax():
    q, scale, am = O.quant_absmax(np.zeros((4, 64), np.uint16))
    assert np.all(q == 0) and scale == 1.0 and am == 0.0
    # a larger given abs-max shrinks the codes: nothing reaches 448
    x = W.normal_bf16((8, 64), 1.0, 3, 1)
    q2, s2, _ = O.quant_absmax(x, np.float32(100.0))
    assert s2 == np.float32(100.0 / 448) and np.max(np.abs(K.e4m3_decode(q2))) < 448


def test_quant_hand_worked():
    # x = [1.6015625, -0.5, 0.001 (bf16: 0.00099945068359375)], abs-max 1.6015625
    # inv = fp32(448 / 1.6015625) = 279.72683..., x*inv = 448, -139.86.., 0.27957..
    # e4m3: 448 -> 0x7E; 139.86 in [128,256): m = rint((139.86/128-1)*8) = 1 -> 144 -> 0x71|0x80
    # 0.27957 in [0.25, 0.5): m = rint((0.27957/0.25-1)*8) = 1 -> 0x29
    x = W.to_bf16_bits(np.array([1.6015625, -0.5, 0.001], np.float32))
    q, scale, am = O.quant_absmax(x)
    assert list(q) == [0x7E, 0xF1, 0x29]
    assert scale == np.float32(1.6015625 / 448)


def test_quant_rows_per_row_scales():
    w = W.normal_bf16((16, 256), 0.02, 4, 1)
    q, s = O.quant_rows(w)
    wv = K.bf16_bits_to_f64(w)
    assert np.array_equal(s, (np.max(np.abs(wv), axis=1) / 448).astype(np.float32))
    for i in range(16):
        assert np.sum(np.isin(q[i], [0x7E, 0xFE])) >= 1


# ----------------------------------------------------------------------------- SiLU / SwiGLU

def test_silu_closed_forms_and_torch():
    assert O.silu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-30, 30, 10001)
    assert np.allclose(O.silu(-x), O.silu(x) - x, atol=1e-12)
    assert np.allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([-1000.0]))[0] == 0.0 and O.silu(np.array([1000.0]))[0] == 1000.0


def test_swiglu_gate_up_placement_and_torch():
    # gate = first H columns, up = last H: a one-hot up column selects the output column
    H = 8
    gu = np.zeros((1, 2 * H), np.float32)
    gu[0, :H] = np.arange(1, H + 1)
    gu[0, H + 5] = 1.0
    h, am = O.swiglu(W.to_bf16_bits(gu))
    hv = K.bf16_bits_to_f64(h)[0]
    assert np.count_nonzero(hv) == 1 and hv[5] != 0
    assert hv[5] == K.bf16_round(6 / (1 + np.exp(-6.0)))
    d = W.block_inputs(16, 128, 256, seed=6)
    gu = W.normal_bf16((16, 512), 2.0, 7, 1)
    h, am = O.swiglu(gu)
    t = bits_to_torch(gu).double()
    want = W.to_bf16_bits((F.silu(t[:, :256]) * t[:, 256:]).float().numpy())
    assert ulp_diff(h, want).max() <= 1
    assert am == np.max(np.abs(K.bf16_bits_to_f64(h)))


# ----------------------------------------------------------------------------- GEMMs

def _frac_gemm(x, w):
    N, Kd = x.shape
    O_ = w.shape[0]
    out = np.empty((N, O_), dtype=object)
    for n in range(N):
        for o in range(O_):
            out[n, o] = sum((Fraction(float(x[n, k])) * Fraction(float(w[o, k])) for k in range(Kd)), Fraction(0))
    return out


def test_gemm_bf16_brute_force_exact_fractions():
    x = W.normal_bf16((3, 24), 1.0, 1, 1)
    w = W.normal_bf16((5, 24), 1.0, 1, 2)  # non-square: a transposed operand cannot fit
    got = K.bf16_bits_to_f64(O.gemm_bf16(x, w))
    ex = _frac_gemm(K.bf16_bits_to_f64(x), K.bf16_bits_to_f64(w))
    want = K.bf16_round(np.array([[float(v) for v in row] for row in ex]))
    assert np.array_equal(got, want)


def test_gemm_bf16_integer_inputs_are_exact_and_match_torch():
    rng = np.random.default_rng(3)
    x = W.to_bf16_bits(rng.integers(-4, 5, (33, 96)).astype(np.float32))
    w = W.to_bf16_bits(rng.integers(-4, 5, (40, 96)).astype(np.float32))
    got = K.bf16_bits_to_f64(O.gemm_bf16(x, w))
    want = (bits_to_torch(x).double() @ bits_to_torch(w).double().T).numpy()
    assert np.all(np.abs(want) < 256)  # exactly representable in bf16
    assert np.array_equal(got, want)


def test_gemm_fp8_matches_torch_and_scales():
    rng = np.random.default_rng(4)
    qx = rng.integers(0, 256, (17, 128)).astype(np.uint8)
    qw = rng.integers(0, 256, (24, 128)).astype(np.uint8)
    qx[(qx & 0x7F) == 0x7F] = 0x11
    qw[(qw & 0x7F) == 0x7F] = 0x22
    sx, sw = np.float32(0.013), np.float32(0.0071)
    got = K.bf16_bits_to_f64(O.gemm_fp8(qx, sx, qw, sw))
    tx = torch.from_numpy(qx).view(torch.float8_e4m3fn).double()
    tw = torch.from_numpy(qw).view(torch.float8_e4m3fn).double()
    s = float(np.float32(np.float64(sx) * np.float64(sw)))
    want = K.bf16_round((tx @ tw.T).numpy() * s)
    assert np.array_equal(got, want)
    # a power-of-two weight scale passes straight through the rounding
    got2 = K.bf16_bits_to_f64(O.gemm_fp8(qx, sx, qw, np.float32(sw * 4)))
    assert np.array_equal(got2, got * 4)


def test_gemm_fp8_brute_force_tiny():
    rng = np.random.default_rng(8)
    qx = rng.integers(0, 0x7E, (2, 16)).astype(np.uint8)
    qw = rng.integers(0x80, 0xFE, (3, 16)).astype(np.uint8)
    ex = _frac_gemm(K.e4m3_decode(qx), K.e4m3_decode(qw))
    s = Fraction(float(np.float32(np.float64(np.float32(0.5)) * np.float64(np.float32(0.25)))))
    want = K.bf16_round(np.array([[float(v * s) for v in row] for row in ex]))
    assert np.array_equal(K.bf16_bits_to_f64(O.gemm_fp8(qx, np.float32(0.5), qw, np.float32(0.25))), want)


# ----------------------------------------------------------------------------- decode

def _brute_decode(x, wg, sg, wu, su, wd, sd):
    """Loops over exact fractions, rounding where the definition rounds."""
    M, C = x.shape
    H = wg.shape[0]
    xv = K.bf16_bits_to_f64(x)
    dg, du, dd = K.e4m3_decode(wg), K.e4m3_decode(wu), K.e4m3_decode(wd)
    y = np.zeros((M, C))
    h = np.zeros((M, H))
    for m in range(M):
        for n in range(H):
            g = sum((Fraction(dg[n, k]) * Fraction(xv[m, k]) for k in range(C)), Fraction(0)) * Fraction(float(sg[n]))
            u = sum((Fraction(du[n, k]) * Fraction(xv[m, k]) for k in range(C)), Fraction(0)) * Fraction(float(su[n]))
            g = K.bf16_round(np.array([float(g)]))[0]
            u = K.bf16_round(np.array([float(u)]))[0]
            h[m, n] = K.bf16_round(np.array([g / (1 + np.exp(-g)) * u]))[0]
        for c in range(C):
            acc = sum((Fraction(dd[c, n]) * Fraction(h[m, n]) for n in range(H)), Fraction(0)) * Fraction(float(sd[c]))
            y[m, c] = K.bf16_round(np.array([float(acc)]))[0]
    return y, h


def test_decode_brute_force():
    d = W.decode_inputs(2, 16, 12, seed=9, w_std=0.02)
    wg, sg = O.quant_rows(d["w_gate"])
    wu, su = O.quant_rows(d["w_up"])
    wd, sd = O.quant_rows(d["w_down"])
    y, h = O.decode_gemv(d["x"], wg, sg, wu, su, wd, sd)
    yb, hb = _brute_decode(d["x"], wg, sg, wu, su, wd, sd)
    assert np.array_equal(K.bf16_bits_to_f64(h), hb)
    assert np.array_equal(K.bf16_bits_to_f64(y), yb)


def _brute_decode_bf16(x, wg, wu, wd):
    """Loops over exact fractions with bf16 weights, rounding where the
    definition rounds."""
    M, C = x.shape
    H = wg.shape[0]
    xv = K.bf16_bits_to_f64(x)
    dg, du, dd = K.bf16_bits_to_f64(wg), K.bf16_bits_to_f64(wu), K.bf16_bits_to_f64(wd)
    y = np.zeros((M, C))
    h = np.zeros((M, H))
    for m in range(M):
        for n in range(H):
            g = K.bf16_round(np.array([float(sum((Fraction(dg[n, k]) * Fraction(xv[m, k]) for k in range(C)),
                                                 Fraction(0)))]))[0]
            u = K.bf16_round(np.array([float(sum((Fraction(du[n, k]) * Fraction(xv[m, k]) for k in range(C)),
                                                 Fraction(0)))]))[0]
            h[m, n] = K.bf16_round(np.array([g / (1 + np.exp(-g)) * u]))[0]
        for c in range(C):
            acc = sum((Fraction(dd[c, n]) * Fraction(h[m, n]) for n in range(H)), Fraction(0))
            y[m, c] = K.bf16_round(np.array([float(acc)]))[0]
    return y, h


def test_decode_bf16_brute_force():
    d = W.decode_inputs(2, 16, 12, seed=19, w_std=0.3)
    y, h = O.decode_gemv_bf16(d["x"], d["w_gate"], d["w_up"], d["w_down"])
    yb, hb = _brute_decode_bf16(d["x"], d["w_gate"], d["w_up"], d["w_down"])
    assert np.array_equal(K.bf16_bits_to_f64(h), hb)
    assert np.array_equal(K.bf16_bits_to_f64(y), yb)


def test_decode_bf16_equals_fp8_decode_on_e4m3_weights_with_unit_scales():
    # bf16 weights that are exactly e4m3 values, and the FP8 decode with all row
    # scales 1: the two definitions coincide
    d = W.decode_inputs(3, 64, 48, seed=20, w_std=2.0)
    codes = {k: K.e4m3_encode(K.bf16_bits_to_f64(d[k])) for k in ("w_gate", "w_up", "w_down")}
    wb = {k: W.to_bf16_bits(K.e4m3_decode(c).astype(np.float32)) for k, c in codes.items()}
    assert all(np.array_equal(K.bf16_bits_to_f64(wb[k]), K.e4m3_decode(codes[k])) for k in wb)
    ones_h, ones_c = np.ones(48, np.float32), np.ones(64, np.float32)
    y8, h8 = O.decode_gemv(d["x"], codes["w_gate"], ones_h, codes["w_up"], ones_h, codes["w_down"], ones_c)
    yb, hb = O.decode_gemv_bf16(d["x"], wb["w_gate"], wb["w_up"], wb["w_down"])
    assert np.array_equal(hb, h8) and np.array_equal(yb, y8)


def test_decode_bf16_zero_gate_gives_zero():
    d = W.decode_inputs(2, 32, 24, seed=21, w_std=0.5)
    zg = np.zeros_like(d["w_gate"])
    y, h = O.decode_gemv_bf16(d["x"], zg, d["w_up"], d["w_down"])
    assert not np.any(K.bf16_bits_to_f64(h)) and not np.any(K.bf16_bits_to_f64(y))


# ----------------------------------------------------------------------------- block invariants

@pytest.mark.parametrize("fp8", [False, True])
def test_block_doubling_down_weight_doubles_output(fp8):
    d = W.block_inputs(32, 128, 256, seed=12)
    a = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=fp8)
    w2 = W.to_bf16_bits((K.bf16_bits_to_f64(d["w_d"]) * 2).astype(np.float32))
    b = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], w2, 1e-5, fp8=fp8)
    assert np.array_equal(K.bf16_bits_to_f64(b["down"]), 2 * K.bf16_bits_to_f64(a["down"]))


def test_block_doubling_up_half_doubles_output_bf16():
    d = W.block_inputs(32, 128, 256, seed=13)
    a = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5)
    wgu = K.bf16_bits_to_f64(d["w_gu"]).copy()
    wgu[256:] *= 2
    b = O.block_forward(d["inp"], d["addend"], d["w_norm"], W.to_bf16_bits(wgu.astype(np.float32)), d["w_d"], 1e-5)
    assert np.array_equal(K.bf16_bits_to_f64(b["h"]), 2 * K.bf16_bits_to_f64(a["h"]))
    assert np.array_equal(K.bf16_bits_to_f64(b["down"]), 2 * K.bf16_bits_to_f64(a["down"]))


@pytest.mark.parametrize("fp8", [False, True])
def test_block_zero_gate_gives_zero_ffn_output(fp8):
    d = W.block_inputs(16, 128, 256, seed=14)
    wgu = d["w_gu"].copy()
    wgu[:256] = 0
    a = O.block_forward(d["inp"], d["addend"], d["w_norm"], wgu, d["w_d"], 1e-5, fp8=fp8)
    assert np.all(K.bf16_bits_to_f64(a["h"]) == 0)
    assert np.all(K.bf16_bits_to_f64(a["down"]) == 0)
    assert np.array_equal(a["next_residual"], a["residual"])


def test_block_rows_are_independent_in_bf16():
    d = W.block_inputs(24, 128, 256, seed=15)
    p = np.random.default_rng(0).permutation(24)
    a = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5)
    b = O.block_forward(d["inp"][p], d["addend"][p], d["w_norm"], d["w_gu"], d["w_d"], 1e-5)
    for k in ("residual", "y", "gu", "h", "down", "next_residual"):
        assert np.array_equal(b[k], a[k][p]), k


def test_block_fp8_close_to_bf16_block():
    # FP8 per-tensor quantisation perturbs the block by a few percent, not more
    d = W.block_inputs(64, 256, 768, seed=16, w_std=0.0)
    a = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5)
    b = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=True)
    da, db = K.bf16_bits_to_f64(a["down"]), K.bf16_bits_to_f64(b["down"])
    assert np.max(np.abs(da - db)) / np.max(np.abs(da)) < 0.1
    assert np.array_equal(a["y"], b["y"]) and a["absmax_y"] == b["absmax_y"]
