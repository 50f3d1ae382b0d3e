"""GPU parity of the backward kernels against the CPU oracle, through the C ABI.

Bit-exact where the result is unique (transposes, quantised codes given the
abs-max, TN products and accumulation on integer-valued operands); within the
stated tolerances where fp32 summation order or the hardware exp/rcp decides
the last bit.  Shapes span several tiles, ragged token counts (padded with
zeros to the GEMM's K granularity) and the largest supported widths.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import codecs as K
from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import (say, dev_bf16, dev_u8, dev_f32, host_bits, host_u8, host_f32, empty_bf16,
                            empty_f32, empty_u8, rel_err, ulp_diff, within_dot_bound)

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_ffn_block_residual_amd as F
    return F


def rand_bits(shape, std, seed):
    rng = np.random.default_rng(seed)
    return W.to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def int_bits(shape, lo, hi, seed):
    rng = np.random.default_rng(seed)
    return W.to_bf16_bits(rng.integers(lo, hi + 1, shape).astype(np.float32))


def rms_bwd_close(got_bits, ref_bits, dres_bits, dy_bits, r_bits, w_bits, rstd):
    """|g - ref| <= one bf16 ulp of ref + 2^-16 of the summed terms'
    magnitudes |dres| + rstd (|dy w| + |xh m|): fp32 rounding of each term
    may move a result that nearly cancels by many ulps of itself."""
    g, ref = K.bf16_bits_to_f64(got_bits), K.bf16_bits_to_f64(ref_bits)
    rs = np.asarray(rstd, np.float64)[:, None]
    xh = K.bf16_bits_to_f64(r_bits) * rs
    gy = K.bf16_bits_to_f64(dy_bits) * K.bf16_bits_to_f64(w_bits)[None, :]
    m = np.sum(gy * xh, axis=1, keepdims=True) / xh.shape[1]
    mag = np.abs(K.bf16_bits_to_f64(dres_bits)) + rs * (np.abs(gy) + np.abs(xh * m))
    return np.all(np.abs(g - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -16 * mag)


def padded_t(x, ld):
    """The oracle transpose with zero columns up to ld."""
    t = O.transpose(x)
    out = np.zeros((t.shape[0], ld), t.dtype)
    out[:, :t.shape[1]] = t
    return out


# ----------------------------------------------------------------------------- transposes

T_SHAPES = [(37, 64, 48), (64, 256, 64), (129, 48, 256), (300, 3584, 384), (1, 16, 128), (0, 32, 128)]


@pytest.mark.parametrize("rows,cols,ld", T_SHAPES)
def test_transpose_bf16_and_codes(F, rows, cols, ld):
    say(f"transpose rows={rows} cols={cols} ld={ld}")
    x = rand_bits((rows, cols), 1.0, rows + cols)
    out = empty_bf16(cols, ld).fill_(7.0)
    F.ffn_transpose(out, dev_bf16(x) if rows else empty_bf16(1, cols), rows, cols, ld, 2)
    q = np.random.default_rng(rows).integers(0, 256, (rows, cols)).astype(np.uint8)
    outq = empty_u8(cols, ld).fill_(9)
    F.ffn_transpose(outq, dev_u8(q) if rows else empty_u8(1, cols), rows, cols, ld, 1)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), padded_t(x, ld))
    assert np.array_equal(host_u8(outq), padded_t(q, ld))


@pytest.mark.parametrize("rows,cols,ld", [(37, 64, 48), (300, 3584, 384), (256, 128, 256)])
def test_quant_transpose(F, rows, cols, ld):
    say(f"quant_transpose rows={rows} cols={cols} ld={ld}")
    x = rand_bits((rows, cols), 3.0, rows * 3 + cols)
    am = O.absmax_of(x)
    for given in (am, np.float32(am * 0.5), np.float32(0.0)):
        qt, q, sc = empty_u8(cols, ld).fill_(5), empty_u8(rows, cols).fill_(6), empty_f32(1)
        F.ffn_quant_transpose(qt, q, sc, dev_bf16(x), dev_f32([given]), rows, cols, ld)
        qt2 = empty_u8(cols, ld).fill_(5)
        F.ffn_quant_transpose(qt2, None, sc, dev_bf16(x), dev_f32([given]), rows, cols, ld)
        torch.cuda.synchronize()
        q_ref, s_ref, _ = O.quant_absmax(x, given)
        assert np.array_equal(host_u8(qt), padded_t(q_ref, ld))
        assert np.array_equal(host_u8(q), q_ref)
        assert torch.equal(qt, qt2)
        assert host_f32(sc)[0] == s_ref


def wide_bits(shape, seed):
    """bf16 values with magnitudes 2^-40 .. 2^3, evenly spread in the exponent,
    random signs and mantissas: quantised against their abs-max they reach
    the e5m2 subnormals and zero as well as its normals."""
    rng = np.random.default_rng(seed)
    v = np.exp2(rng.uniform(-40.0, 3.0, shape)) * rng.choice([-1.0, 1.0], shape)
    return W.to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("rows,cols,ld", [(37, 64, 48), (300, 3584, 384), (256, 128, 256)])
def test_quant_transpose_e5m2(F, rows, cols, ld):
    say(f"quant_transpose e5m2 rows={rows} cols={cols} ld={ld}")
    x = wide_bits((rows, cols), rows + 5 * cols)
    am = O.absmax_of(x)
    for given in (am, np.float32(am * 0.25), np.float32(0.0)):
        qt, q, sc = empty_u8(cols, ld).fill_(5), empty_u8(rows, cols).fill_(6), empty_f32(1)
        F.ffn_quant_transpose(qt, q, sc, dev_bf16(x), dev_f32([given]), rows, cols, ld, code_dtype=F.FFN_E5M2)
        torch.cuda.synchronize()
        q_ref, s_ref, _ = O.quant_absmax(x, given, "e5m2")
        codes = host_u8(q)
        assert np.array_equal(host_u8(qt), padded_t(q_ref, ld))
        assert np.array_equal(codes, q_ref)
        assert host_f32(sc)[0] == s_ref
        if given == am:
            # the spread reaches every e5m2 binade: subnormal codes and zeros
            assert np.any(((codes & 0x7C) == 0) & ((codes & 0x03) != 0)) and np.any((codes & 0x7F) == 0)
        if given == np.float32(am * 0.25):
            # values beyond the given abs-max saturate at +-57344 (0x7B / 0xFB)
            assert np.any((codes & 0x7F) == 0x7B) and not np.any((codes & 0x7C) == 0x7C)


# ----------------------------------------------------------------------------- TN products

MM_SHAPES = [(1, 128, 128), (37, 256, 640), (300, 384, 256), (513, 128, 1024)]


@pytest.mark.parametrize("M,N,Kd", MM_SHAPES)
def test_matmul_tn_integer_exact_and_accumulate(F, M, N, Kd):
    say(f"matmul_tn integer M={M} N={N} K={Kd}")
    a, b = int_bits((M, Kd), -2, 2, M + Kd), int_bits((N, Kd), -2, 2, N + 1)
    out = empty_bf16(M, N).fill_(3.0)
    F.ffn_matmul_tn(out, dev_bf16(a), None, dev_bf16(b), None, F.FFN_BF16, 0, M, N, Kd)
    # accumulation onto small integers: every partial sum exact in fp32, one rounding
    acc0 = int_bits((M, N), -8, 8, M * 7)
    acc = dev_bf16(acc0)
    a_s, b_s = int_bits((M, Kd), -1, 1, 5), int_bits((N, Kd), -1, 1, 6)
    F.ffn_matmul_tn(acc, dev_bf16(a_s), None, dev_bf16(b_s), None, F.FFN_BF16, 1, M, N, Kd)
    # e4m3 codes of small integers with unit scales
    qa = K.e4m3_encode(K.bf16_bits_to_f64(a_s))
    qb = K.e4m3_encode(K.bf16_bits_to_f64(b_s))
    one = dev_f32([1.0])
    out8 = empty_bf16(M, N).fill_(3.0)
    F.ffn_matmul_tn(out8, dev_u8(qa), one, dev_u8(qb), one, F.FFN_E4M3, 0, M, N, Kd)
    acc8 = dev_bf16(acc0)
    F.ffn_matmul_tn(acc8, dev_u8(qa), one, dev_u8(qb), one, F.FFN_E4M3, 1, M, N, Kd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), O.matmul_tn(a, b))
    want_acc = O.matmul_tn(a_s, b_s, accumulate=acc0)
    assert np.array_equal(host_bits(acc), want_acc)
    assert np.array_equal(host_bits(out8), O.matmul_tn(qa, qb, 1.0, 1.0))
    assert np.array_equal(host_bits(acc8), want_acc)


@pytest.mark.parametrize("M,N,Kd", [(37, 256, 640), (300, 384, 1024)])
def test_matmul_tn_random_fp8_scaled_accumulate(F, M, N, Kd):
    say(f"matmul_tn fp8 random M={M} N={N} K={Kd}")
    a, b = rand_bits((M, Kd), 1.0, 11), rand_bits((N, Kd), 1.0, 12)
    qa, sa, _ = O.quant_absmax(a)
    qb, sb, _ = O.quant_absmax(b)
    acc0 = rand_bits((M, N), 50.0, 13)
    out = dev_bf16(acc0)
    F.ffn_matmul_tn(out, dev_u8(qa), dev_f32([sa]), dev_u8(qb), dev_f32([sb]), F.FFN_E4M3, 1, M, N, Kd)
    torch.cuda.synchronize()
    s = np.float64(np.float32(np.float64(sa) * np.float64(sb)))
    exact = (K.e4m3_decode(qa) @ K.e4m3_decode(qb).T) * s + K.bf16_bits_to_f64(acc0)
    mag = (np.abs(K.e4m3_decode(qa)) @ np.abs(K.e4m3_decode(qb)).T) * s + np.abs(K.bf16_bits_to_f64(acc0))
    assert np.all(within_dot_bound(host_bits(out), exact, mag))


@pytest.mark.parametrize("M,N,Kd", [(4300, 4096, 256), (6900, 4864, 512)])
def test_matmul_tn_uneven_rounds_exact(F, M, N, Kd):
    """Output tile counts just past one and two rounds of 256 CUs (17 x 16 =
    272 and 27 x 19 = 513 tiles of 256 x 256): the persistent grid deals them
    over 136 and 176 workgroups that take one to three tiles each, a ragged
    last row of tiles included.  Integer-valued e4m3 codes, exact sums."""
    say(f"matmul_tn uneven rounds M={M} N={N} K={Kd}")
    rng = np.random.default_rng(M + N)
    qa = K.e4m3_encode(rng.integers(-3, 4, (M, Kd)).astype(np.float64))
    qb = K.e4m3_encode(rng.integers(-3, 4, (N, Kd)).astype(np.float64))
    one = dev_f32([1.0])
    out = empty_bf16(M, N).fill_(3.0)
    F.ffn_matmul_tn(out, dev_u8(qa), one, dev_u8(qb), one, F.FFN_E4M3, 0, M, N, Kd)
    # one workgroup per tile: the same products
    out_t = empty_bf16(M, N).fill_(3.0)
    F.ffn_matmul_tn(out_t, dev_u8(qa), one, dev_u8(qb), one, F.FFN_E4M3, F.FFN_TN_TILE_GRID, M, N, Kd)
    torch.cuda.synchronize()
    exact = K.e4m3_decode(qa) @ K.e4m3_decode(qb).T
    assert np.array_equal(host_bits(out), O.f64_to_bf16_bits(exact))
    assert torch.equal(out_t, out)


@pytest.mark.parametrize("M,N,Kd", MM_SHAPES)
def test_matmul_tn_e5m2_gradient_exact(F, M, N, Kd):
    """a in e5m2, b in e4m3 (FFN_E5M2): integer-valued codes and e5m2
    subnormals times small integers, whose fp32 sums are exact, so the bf16
    result is unique; plain and accumulating."""
    say(f"matmul_tn e5m2 exact M={M} N={N} K={Kd}")
    rng = np.random.default_rng(M * 3 + Kd)
    # e5m2 codes of -4..4 and of the subnormals +-2^-16 .. +-3 * 2^-16
    ints = K.e5m2_encode(rng.integers(-4, 5, (M, Kd)).astype(np.float64))
    subn = rng.choice(np.array([0x00, 0x01, 0x02, 0x03, 0x81, 0x82, 0x83], np.uint8), (M, Kd))
    qb = K.e4m3_encode(rng.integers(-2, 3, (N, Kd)).astype(np.float64))
    one = dev_f32([1.0])
    acc0 = int_bits((M, N), -8, 8, M + 99)
    for qa in (ints, subn):
        out = empty_bf16(M, N).fill_(3.0)
        F.ffn_matmul_tn(out, dev_u8(qa), one, dev_u8(qb), one, F.FFN_E5M2, 0, M, N, Kd)
        acc = dev_bf16(acc0)
        F.ffn_matmul_tn(acc, dev_u8(qa), one, dev_u8(qb), one, F.FFN_E5M2, 1, M, N, Kd)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), O.matmul_tn(qa, qb, 1.0, 1.0, a_fmt="e5m2"))
        assert np.array_equal(host_bits(acc), O.matmul_tn(qa, qb, 1.0, 1.0, accumulate=acc0, a_fmt="e5m2"))


@pytest.mark.parametrize("M,N,Kd", [(37, 256, 640), (300, 384, 1024)])
def test_matmul_tn_random_e5m2_scaled_accumulate(F, M, N, Kd):
    say(f"matmul_tn e5m2 random M={M} N={N} K={Kd}")
    a, b = wide_bits((M, Kd), 21), rand_bits((N, Kd), 1.0, 22)
    qa, sa, _ = O.quant_absmax(a, fmt="e5m2")
    qb, sb, _ = O.quant_absmax(b)
    acc0 = rand_bits((M, N), 50.0, 23)
    out = dev_bf16(acc0)
    F.ffn_matmul_tn(out, dev_u8(qa), dev_f32([sa]), dev_u8(qb), dev_f32([sb]), F.FFN_E5M2, 1, M, N, Kd)
    torch.cuda.synchronize()
    s = np.float64(np.float32(np.float64(sa) * np.float64(sb)))
    da, db = K.e5m2_decode(qa), K.e4m3_decode(qb)
    exact = (da @ db.T) * s + K.bf16_bits_to_f64(acc0)
    mag = (np.abs(da) @ np.abs(db).T) * s + np.abs(K.bf16_bits_to_f64(acc0))
    assert np.all(within_dot_bound(host_bits(out), exact, mag))


# ----------------------------------------------------------------------------- SwiGLU backward

@pytest.mark.parametrize("N,H", [(64, 768), (37, 1000), (300, 256), (1, 8), (0, 64)])
def test_swiglu_bwd(F, N, H):
    say(f"swiglu_bwd N={N} H={H}")
    gu = rand_bits((N, 2 * H), 3.0, N + H)
    dh = rand_bits((N, H), 1.0, N * 2 + H)
    dgu, am = empty_bf16(max(N, 1), 2 * H), empty_f32(1).fill_(5.0)
    gdev = dev_bf16(gu) if N else empty_bf16(1, 2 * H)
    ddev = dev_bf16(dh) if N else empty_bf16(1, H)
    F.ffn_swiglu_bwd(dgu, am, ddev, gdev, N, H)
    # in place over gu (the trainer writes dMlpUp over MlpUp)
    F.ffn_swiglu_bwd(gdev, None, ddev, gdev, N, H)
    torch.cuda.synchronize()
    if N == 0:
        assert host_f32(am)[0] == 0.0
        return
    ref, am_ref = O.swiglu_bwd(dh, gu)
    got = host_bits(dgu)
    d = ulp_diff(got, ref)
    assert d.max() <= 2 and np.mean(d != 0) < 1e-2
    assert host_f32(am)[0] == np.max(np.abs(K.bf16_bits_to_f64(got)))
    assert np.array_equal(host_bits(gdev), got)


FUSED_SHAPES = [(37, 256, 640, "bf16"), (300, 384, 256, "e4m3"), (513, 128, 1024, "e5m2"), (1, 128, 128, "e4m3"),
                (200, 640, 384, "bf16"), (0, 128, 128, "e4m3")]


@pytest.mark.parametrize("M,H,Kd,dt", FUSED_SHAPES)
@pytest.mark.parametrize("in_place", [False, True])
def test_matmul_tn_swiglu_bwd_equals_two_calls(F, M, H, Kd, dt, in_place):
    """The fused data gradient + SwiGLU backward equals ffn_matmul_tn then
    ffn_swiglu_bwd bit for bit (dgu and its abs-max), in place over gu too;
    with integer-valued operands dh is exact and dgu is the oracle's
    swiglu_bwd of it up to the hardware exp's last bits."""
    say(f"matmul_tn_swiglu_bwd M={M} H={H} K={Kd} {dt} in_place={in_place}")
    rng = np.random.default_rng(M + H + Kd)
    code = {"bf16": F.FFN_BF16, "e4m3": F.FFN_E4M3, "e5m2": F.FFN_E5M2}[dt]
    Mr = max(M, 1)
    ia = rng.integers(-2, 3, (Mr, Kd)).astype(np.float64)
    ib = rng.integers(-2, 3, (H, Kd)).astype(np.float64)
    if dt == "bf16":
        a, b = dev_bf16(W.to_bf16_bits(ia.astype(np.float32))), dev_bf16(W.to_bf16_bits(ib.astype(np.float32)))
        sa = sb = None
        dh_exact = ia @ ib.T
    else:
        qa = K.e5m2_encode(ia) if dt == "e5m2" else K.e4m3_encode(ia)
        qb = K.e4m3_encode(ib)
        a, b = dev_u8(qa), dev_u8(qb)
        sa, sb = dev_f32([0.5]), dev_f32([0.25])
        dh_exact = (ia @ ib.T) * 0.125
    gu = rand_bits((Mr, 2 * H), 2.0, M * 7 + H)
    dh = empty_bf16(Mr, H)
    F.ffn_matmul_tn(dh, a, sa, b, sb, code, 0, M, H, Kd)
    ref, am_ref = empty_bf16(Mr, 2 * H).fill_(9.0), empty_f32(1).fill_(5.0)
    F.ffn_swiglu_bwd(ref, am_ref, dh, dev_bf16(gu), M, H)
    gdev = dev_bf16(gu)
    out = gdev if in_place else empty_bf16(Mr, 2 * H).fill_(9.0)
    am = empty_f32(1).fill_(5.0)
    out_t, am_t = empty_bf16(Mr, 2 * H).fill_(9.0), empty_f32(1).fill_(5.0)
    F.ffn_matmul_tn_swiglu_bwd(out_t, am_t, a, sa, b, sb, dev_bf16(gu), code, M, H, Kd, flags=F.FFN_TN_TILE_GRID)
    F.ffn_matmul_tn_swiglu_bwd(out, am, a, sa, b, sb, gdev, code, M, H, Kd)
    torch.cuda.synchronize()
    assert host_f32(am)[0] == host_f32(am_ref)[0] and host_f32(am_t)[0] == host_f32(am_ref)[0]
    assert torch.equal(out_t[:M], ref[:M])
    if M == 0:
        assert host_f32(am)[0] == 0.0
        return
    assert torch.equal(out[:M], ref[:M])
    dgu_o, _ = O.swiglu_bwd(O.f64_to_bf16_bits(dh_exact[:M]), gu[:M])
    d = ulp_diff(host_bits(out[:M]), dgu_o)
    assert d.max() <= 2 and np.mean(d != 0) < 1e-2


def test_matmul_tn_swiglu_bwd_full_size(F):
    """At the Llama-8B shape (M=4096 tokens, H=14336, K=C=4096, e4m3) the
    fused kernel equals the two calls bit for bit."""
    M, H, Kd = 4096, 14336, 4096
    say(f"matmul_tn_swiglu_bwd full size M={M} H={H} K={Kd}")
    rng = np.random.default_rng(11)
    a = torch.from_numpy(rng.integers(0, 256, (M, Kd), dtype=np.uint8)).cuda()
    b = torch.from_numpy(rng.integers(0, 256, (H, Kd), dtype=np.uint8)).cuda()
    # no NaN codes (0x7F, 0xFF) in the operands
    a[(a & 0x7F) == 0x7F] = 0x40
    b[(b & 0x7F) == 0x7F] = 0x40
    sa, sb = dev_f32([2.0 ** -6]), dev_f32([2.0 ** -6])
    gu = (torch.randn(M, 2 * H, device="cuda", generator=torch.Generator("cuda").manual_seed(3)) * 2).bfloat16()
    dh = empty_bf16(M, H)
    F.ffn_matmul_tn(dh, a, sa, b, sb, F.FFN_E4M3, 0, M, H, Kd)
    ref, am_ref = empty_bf16(M, 2 * H), empty_f32(1)
    F.ffn_swiglu_bwd(ref, am_ref, dh, gu, M, H)
    out, am = empty_bf16(M, 2 * H), empty_f32(1)
    F.ffn_matmul_tn_swiglu_bwd(out, am, a, sa, b, sb, gu, F.FFN_E4M3, M, H, Kd)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert host_f32(am)[0] == host_f32(am_ref)[0]


# ----------------------------------------------------------------------------- RMSNorm backward

@pytest.mark.parametrize("N,C", [(64, 256), (37, 3584), (300, 4096), (5, 8192), (1, 8), (1000, 384)])
def test_rmsnorm_bwd(F, N, C):
    say(f"rmsnorm_bwd N={N} C={C}")
    d = W.block_inputs(N, C, 128, seed=N + C)
    r = O.residual_add(d["inp"], d["addend"])
    rstd = O.rms_rstd(r, 1e-5)
    dy = rand_bits((N, C), 1.0, N + 3)
    dres = rand_bits((N, C), 0.5, N + 4)
    dw0 = np.random.default_rng(N).standard_normal(C).astype(np.float32)
    dinp, dw, am = empty_bf16(N, C), dev_f32(dw0), empty_f32(1)
    scratch = empty_f32(max(F.ffn_rmsnorm_bwd_scratch_bytes(N, C), 4) // 4)
    rd, dyd, wd, rsd = dev_bf16(r), dev_bf16(dy), dev_bf16(d["w_norm"]), dev_f32(rstd)
    F.ffn_rmsnorm_bwd(dinp, dw, scratch, dev_bf16(dres), dyd, rd, wd, rsd, am, N, C)
    # in place over the residual gradient, accumulating into the same dweight
    dres_dev = dev_bf16(dres)
    F.ffn_rmsnorm_bwd(dres_dev, dw, scratch, dres_dev, dyd, rd, wd, rsd, None, N, C)
    torch.cuda.synchronize()
    ref, dw_ref, am_ref = O.rmsnorm_bwd(dres, dy, r, d["w_norm"], rstd, dw0)
    got = host_bits(dinp)
    # fp32 products and the row sum in another order than the oracle's fp64
    assert rms_bwd_close(got, ref, dres, dy, r, d["w_norm"], rstd)
    assert np.mean(ulp_diff(got, ref) != 0) < 5e-3
    assert rel_err(got, ref) < 2e-2
    assert host_f32(am)[0] == np.max(np.abs(K.bf16_bits_to_f64(got)))
    assert np.array_equal(host_bits(dres_dev), got)
    _, dw2_ref, _ = O.rmsnorm_bwd(dres, dy, r, d["w_norm"], rstd, dw_ref)
    g_dw = host_f32(dw)
    # fp32 sums over N rows in another order: bounded by the terms' magnitudes
    xh = K.bf16_bits_to_f64(r) * rstd.astype(np.float64)[:, None]
    mag = 2 * np.sum(np.abs(K.bf16_bits_to_f64(dy) * xh), axis=0) + np.abs(dw0)
    assert np.all(np.abs(g_dw - dw2_ref) <= 2.0 ** -16 * mag + 1e-30)


# ----------------------------------------------------------------------------- the block

def _run_block(F, N, C, H, fp8, seed, w_std=0.1, in_place=True, grad_dtype="e4m3", fuse=False):
    """fuse=False: the two-call form, which keeps dh for the stage checks."""
    from transformer_ffn_block_residual_amd import block
    d = W.block_inputs(N, C, H, seed=seed, w_std=w_std)
    pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
    pb.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    bb = block.BackwardBlock(pb, in_place=in_place, grad_dtype=grad_dtype, fuse_swiglu_bwd=fuse)
    d_out = rand_bits((N, C), 1.0, seed + 1)
    bb.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
    d_out_dev = dev_bf16(d_out)
    bb.backward(d_out_dev)
    torch.cuda.synchronize()
    return d, pb, bb, d_out


@pytest.mark.parametrize("N,C,H,fp8", [(64, 256, 768, False), (200, 384, 256, False), (200, 384, 256, True),
                                       (129, 256, 640, True)])
def test_block_backward_against_the_oracle(F, N, C, H, fp8):
    say(f"block backward N={N} C={C} H={H} fp8={fp8}")
    d, pb, bb, d_out = _run_block(F, N, C, H, fp8, seed=N + H)
    fwd = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=fp8)
    ref = O.block_backward(fwd, d_out, d["w_norm"], d["w_gu"], d["w_d"], fp8=fp8)
    tol = 2e-2 if not fp8 else 3e-2
    # conditional checks: each stage on the GPU's own upstream tensors
    g_dh = host_bits(bb.dh)
    g_dgu = host_bits(bb.dgu)
    g_dy = host_bits(bb.dy)
    gu_ref = O.gemm_bf16(host_bits(pb.y), d["w_gu"]) if not fp8 else None
    if not fp8:
        assert np.array_equal(host_bits(pb.h), O.swiglu(gu_ref)[0]) or rel_err(host_bits(pb.h), O.swiglu(gu_ref)[0]) < 1e-2
        dgu_cond, _ = O.swiglu_bwd(g_dh, gu_ref)
        assert rel_err(g_dgu, dgu_cond) < 2e-2
        lin = O.linear_bwd(g_dgu, host_bits(pb.y), d["w_gu"])
        assert rel_err(g_dy, lin["dx"]) < 1e-2
    dres_cond, dwn_cond, _ = O.rmsnorm_bwd(d_out, g_dy, host_bits(pb.r), d["w_norm"], host_f32(pb.rstd))
    assert rel_err(host_bits(bb.d_res), dres_cond) < 1e-2
    assert np.max(np.abs(host_f32(bb.dw_norm) - dwn_cond)) <= 1e-4 * np.max(np.abs(dwn_cond))
    # end to end against the oracle's own chain (its own quantisation decisions
    # for FP8: measured against each tensor's max, as the forward's FP8 chain)
    def normwise(g, r):
        g, r = K.bf16_bits_to_f64(g), K.bf16_bits_to_f64(r)
        return np.max(np.abs(g - r)) / np.max(np.abs(r))
    for name, got in (("dh", g_dh), ("dgu", g_dgu), ("dy", g_dy), ("d_residual", host_bits(bb.d_res)),
                      ("dw_d", host_bits(bb.dw_d)), ("dw_gu", host_bits(bb.dw_gu))):
        err = rel_err(got, ref[name]) if not fp8 else normwise(got, ref[name])
        assert err < tol, (name, err)
    dwn = host_f32(bb.dw_norm)
    assert np.max(np.abs(dwn - ref["dw_norm"])) <= tol * np.max(np.abs(ref["dw_norm"]))


@pytest.mark.parametrize("N,C,H", [(200, 384, 256), (129, 256, 640)])
def test_block_backward_e5m2_gradients(F, N, C, H):
    """The FP8 backward with e5m2 gradient codes.  Stage by stage on the
    GPU's own upstream tensors: the gradient codes and scales exactly, each TN
    product within the dot bound of its exact value; then end to end against
    the oracle's e5m2 chain, normwise within 6e-2 (twice the e4m3 chain's
    3e-2: e5m2 keeps one mantissa bit less)."""
    say(f"block backward e5m2 N={N} C={C} H={H}")
    d, pb, bb, d_out = _run_block(F, N, C, H, True, seed=N + H + 1, in_place=False, grad_dtype="e5m2")
    dec5, dec4 = K.e5m2_decode, K.e4m3_decode
    f32 = lambda v: np.float64(np.float32(v))

    def tn_close(got, a_codes, b_codes, sa, sb):
        s = f32(np.float64(sa) * np.float64(sb))
        A, Bm = dec5(a_codes), dec4(b_codes)
        return np.all(within_dot_bound(got, (A @ Bm.T) * s, (np.abs(A) @ np.abs(Bm).T) * s))

    # output gradient: abs-max computed here, codes in both layouts
    q_dout, s_dout, _ = O.quant_absmax(d_out, fmt="e5m2")
    assert np.array_equal(host_u8(bb.qdout), q_dout) and host_f32(bb.s_dout)[0] == s_dout
    assert np.array_equal(host_u8(bb.dout_t), padded_t(q_dout, bb.Np))
    wd, s_d = host_u8(pb.w_d), host_f32(pb.s_d)[0]           # [C, H] e4m3
    g_dh = host_bits(bb.dh)
    assert tn_close(g_dh, q_dout, O.transpose(wd), s_dout, s_d)
    qh, s_h = host_u8(pb.qh), host_f32(pb.s_h)[0]
    assert tn_close(host_bits(bb.dw_d), O.transpose(q_dout), O.transpose(qh), s_dout, s_h)
    # dMlpUp from the GPU's dh and gu, its abs-max, its e5m2 codes
    g_dgu = host_bits(bb.dgu)
    dgu_ref, _ = O.swiglu_bwd(g_dh, host_bits(bb.gu))
    assert rel_err(g_dgu, dgu_ref) < 1e-2
    am_dgu = host_f32(bb.am_dgu)[0]
    assert am_dgu == O.absmax_of(g_dgu)
    q_dgu, s_dgu, _ = O.quant_absmax(g_dgu, am_dgu, "e5m2")
    assert np.array_equal(host_u8(bb.qdgu), q_dgu) and host_f32(bb.s_dgu)[0] == s_dgu
    assert np.array_equal(host_u8(bb.dgu_t), padded_t(q_dgu, bb.Np))
    wgu, s_gu = host_u8(pb.w_gu), host_f32(pb.s_gu)[0]       # [2H, C] e4m3
    assert tn_close(host_bits(bb.dy), q_dgu, O.transpose(wgu), s_dgu, s_gu)
    qy, s_y = host_u8(pb.qy), host_f32(pb.s_y)[0]
    assert tn_close(host_bits(bb.dw_gu), O.transpose(q_dgu), O.transpose(qy), s_dgu, s_y)
    # end to end against the oracle's e5m2 chain
    fwd = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=True)
    ref = O.block_backward(fwd, d_out, d["w_norm"], d["w_gu"], d["w_d"], fp8=True, grad_fmt="e5m2")

    def normwise(g, r):
        g, r = K.bf16_bits_to_f64(g), K.bf16_bits_to_f64(r)
        return np.max(np.abs(g - r)) / np.max(np.abs(r))
    for name, got in (("dh", g_dh), ("dgu", g_dgu), ("dy", host_bits(bb.dy)),
                      ("d_residual", host_bits(bb.d_res)), ("dw_d", host_bits(bb.dw_d)),
                      ("dw_gu", host_bits(bb.dw_gu))):
        err = normwise(got, ref[name])
        assert err < 6e-2, (name, err)
    assert np.max(np.abs(host_f32(bb.dw_norm) - ref["dw_norm"])) <= 6e-2 * np.max(np.abs(ref["dw_norm"]))


@pytest.mark.parametrize("fp8,grad,in_place", [(False, "e4m3", True), (True, "e4m3", False), (True, "e5m2", True)])
def test_block_backward_fused_swiglu_equals_two_calls(F, fp8, grad, in_place):
    """BackwardBlock with the fused data gradient + SwiGLU backward gives
    every output of the two-call form bit for bit."""
    say(f"block backward fused vs two calls fp8={fp8} grad={grad} in_place={in_place}")
    N, C, H = 200, 384, 640
    res = []
    for fuse in (False, True):
        d, pb, bb, d_out = _run_block(F, N, C, H, fp8, seed=77, in_place=in_place, grad_dtype=grad, fuse=fuse)
        res.append({n: getattr(bb, n).clone() for n in ("dgu", "dy", "d_res", "dw_d", "dw_gu", "dw_norm",
                                                           "am_dgu", "am_dres")})
    for n in res[0]:
        assert torch.equal(res[0][n], res[1][n]), n


@pytest.mark.parametrize("fp8,grad,in_place,fuse", [(False, "e4m3", True, True), (False, "e4m3", False, False),
                                                    (True, "e4m3", True, True), (True, "e5m2", False, True),
                                                    (True, "e4m3", False, False)])
def test_block_backward_concurrent_equals_serial(F, fp8, grad, in_place, fuse):
    """The two-stream schedule (weight gradients beside the data gradients,
    one workgroup per tile) gives every output of the serial one bit for bit,
    over two accumulating calls."""
    say(f"block backward concurrent vs serial fp8={fp8} grad={grad} in_place={in_place} fuse={fuse}")
    from transformer_ffn_block_residual_amd import block
    N, C, H = 300, 384, 640
    d = W.block_inputs(N, C, H, seed=88, w_std=0.1)
    d_out = dev_bf16(rand_bits((N, C), 1.0, 89))
    res = []
    for conc in (False, True):
        pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
        pb.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
        bb = block.BackwardBlock(pb, in_place=in_place, grad_dtype=grad, fuse_swiglu_bwd=fuse, concurrent=conc)
        for _ in range(2):
            bb.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
            bb.backward(d_out)
        torch.cuda.synchronize()
        res.append({n: getattr(bb, n).clone() for n in ("dgu", "dy", "d_res", "dw_d", "dw_gu", "dw_norm",
                                                           "am_dgu", "am_dres")})
    for n in res[0]:
        assert torch.equal(res[0][n], res[1][n]), n


@pytest.mark.parametrize("fp8,grad,in_place,fuse,conc", [(True, "e4m3", True, True, False),
                                                         (True, "e5m2", False, False, False),
                                                         (True, "e4m3", True, True, True),
                                                         (False, "e4m3", True, True, False)])
def test_block_backward_zero_once_equals_default(F, fp8, grad, in_place, fuse, conc):
    """The zero-once abs-max form of the backward (the SwiGLU and RMSNorm
    backwards accumulate into zeroed words; the quantiser of dMlpUp and the
    RMSNorm backward clear each other's word) gives every gradient, scale and
    d_res abs-max of the default form bit for bit, over three calls whose
    output gradients shrink and grow again (a word left uncleared would show
    in the next call's scale), and leaves dMlpUp's word at zero."""
    say(f"block backward zero-once fp8={fp8} grad={grad} in_place={in_place} fuse={fuse} conc={conc}")
    from transformer_ffn_block_residual_amd import block
    N, C, H = 300, 384, 640
    d = W.block_inputs(N, C, H, seed=91, w_std=0.1)
    outs = [dev_bf16(rand_bits((N, C), std, 92 + k)) for k, std in enumerate((1.0, 0.01, 3.0))]
    blocks = []
    for zo in (False, True):
        pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
        pb.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
        blocks.append(block.BackwardBlock(pb, in_place=in_place, grad_dtype=grad, fuse_swiglu_bwd=fuse,
                                          concurrent=conc, zero_once=zo))
    names = ["dgu", "dy", "d_res", "dw_d", "dw_gu", "dw_norm"] + (["s_dgu", "am_dres"] if fp8 else [])
    for k, d_out in enumerate(outs):
        got = []
        for bb in blocks:
            bb.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
            bb.backward(d_out)
            torch.cuda.synchronize()
            got.append({n: getattr(bb, n).clone() for n in names})
        for n in names:
            assert torch.equal(got[0][n], got[1][n]), (k, n)
        zo = blocks[1]
        assert host_f32(zo.am_dgu)[0] == 0.0, k
        if fp8:
            assert host_f32(zo.am_dres)[0] > 0.0, k
        else:
            assert host_f32(zo.am_dres)[0] == 0.0 and host_f32(zo.am_tab).max() == 0.0, k


def test_block_backward_accumulates_weight_gradients(F):
    say("block backward twice")
    N, C, H = 128, 256, 384
    d, pb, bb, d_out = _run_block(F, N, C, H, False, seed=3)
    one = [host_bits(bb.dw_d), host_bits(bb.dw_gu), host_f32(bb.dw_norm)]
    bb.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
    bb.backward(dev_bf16(d_out))
    torch.cuda.synchronize()
    two = [host_bits(bb.dw_d), host_bits(bb.dw_gu), host_f32(bb.dw_norm)]
    for a, b in zip(one[:2], two[:2]):
        # bf16(g + bf16(g)) against 2g: one more rounding
        assert rel_err(b, O.f64_to_bf16_bits(2 * K.bf16_bits_to_f64(a))) < 1e-2
    assert np.allclose(two[2], 2 * one[2], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("fp8", [False, True])
def test_block_backward_remakes_weight_transposes_after_a_weight_update(F, fp8):
    """The transposed weights are cached across backward calls; new weights
    (load_weights, or an in-place update declared with weights_changed) must
    be seen by the next backward exactly as by a block built with them."""
    say(f"block backward after a weight update fp8={fp8}")
    from transformer_ffn_block_residual_amd import block
    N, C, H = 96, 256, 384
    d1 = W.block_inputs(N, C, H, seed=21, w_std=0.1)
    d2 = W.block_inputs(N, C, H, seed=22, w_std=0.1)
    d_out = dev_bf16(rand_bits((N, C), 1.0, 23))
    inp, add = dev_bf16(d1["inp"]), dev_bf16(d1["addend"])

    def grads(bb):
        bb.zero_grads()
        bb.forward(inp, add)
        bb.backward(d_out)
        torch.cuda.synchronize()
        return [t.clone() for t in (bb.d_res, bb.dw_d, bb.dw_gu, bb.dw_norm)]

    pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
    pb.load_weights(d1["w_norm"], d1["w_gu"], d1["w_d"])
    bb = block.BackwardBlock(pb)
    grads(bb)
    pb.load_weights(d2["w_norm"], d2["w_gu"], d2["w_d"])
    got = grads(bb)
    fresh_pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
    fresh_pb.load_weights(d2["w_norm"], d2["w_gu"], d2["w_d"])
    want = grads(block.BackwardBlock(fresh_pb))
    for a, b in zip(got, want):
        assert torch.equal(a, b)
    if fp8:
        return
    # an in-place update of the bf16 weights, declared
    for t in (pb.w_gu, pb.w_d, fresh_pb.w_gu, fresh_pb.w_d):
        t.mul_(0.5)
    pb.weights_changed()
    got = grads(bb)
    want = grads(block.BackwardBlock(fresh_pb))
    for a, b in zip(got, want):
        assert torch.equal(a, b)


@pytest.mark.parametrize("fp8", [False, True])
def test_block_backward_out_of_place_and_given_absmax(F, fp8):
    say(f"block backward out of place fp8={fp8}")
    from transformer_ffn_block_residual_amd import block
    N, C, H = 96, 256, 384
    d = W.block_inputs(N, C, H, seed=9, w_std=0.1)
    d_out = dev_bf16(rand_bits((N, C), 1.0, 10))
    # the second run takes d_out's abs-max from outside, as from its producer
    am = empty_f32(1)
    F.ffn_quant_absmax(empty_u8(N * C), empty_f32(1), am, d_out, N * C, 1)
    res = []
    for in_place in (True, False):
        pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
        pb.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
        bb = block.BackwardBlock(pb, in_place=in_place)
        bb.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
        gu0 = bb.gu.clone()
        bb.backward(d_out, d_out_absmax=None if in_place else am)
        torch.cuda.synchronize()
        res.append((bb.dgu.clone(), bb.d_res.clone(), bb.dw_d.clone(), bb.dw_gu.clone(), bb.dw_norm.clone()))
        if not in_place:
            assert torch.equal(bb.gu, gu0)
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("grad", ["e4m3", "e5m2"])
def test_block_backward_full_size_sampled(F, grad):
    """FP8 block backward at N=4096, C=4096, H=14336: each GEMM output checked
    on sampled entries against the exact product of the GPU's own codes, the
    SwiGLU and RMSNorm backward on sampled rows.  grad: the gradients' codes."""
    N, C, H = 4096, 4096, 14336
    say(f"block backward full size N={N} C={C} H={H} fp8, {grad} gradients")
    from transformer_ffn_block_residual_amd import block
    d = W.block_inputs(N, C, H, seed=1004, w_std=0.02)
    pb = block.PrefillBlock(N, C, H, 1e-5, True)
    pb.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    bb = block.BackwardBlock(pb, grad_dtype=grad, fuse_swiglu_bwd=False)
    gdec = K.e5m2_decode if grad == "e5m2" else K.e4m3_decode
    gu_keep = empty_bf16(N, 2 * H)
    bb.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
    gu_keep.copy_(bb.gu)
    d_out = rand_bits((N, C), 1.0, 77)
    bb.backward(dev_bf16(d_out))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, N - 1, 255, 256], rng.integers(0, N, 12)]))
    qdout = host_u8(bb.qdout)
    wd = host_u8(pb.w_d).reshape(C, H)
    s = float(np.float32(host_f32(bb.s_dout)[0] * host_f32(pb.s_d)[0]))
    # dh rows: sum_c dec(qdout[n, c]) dec(Wd[c, h]) * s
    dq = gdec(qdout[rows])
    wdec = K.e4m3_decode(wd)
    exact = dq @ wdec * s
    mag = np.abs(dq) @ np.abs(wdec) * abs(s)
    assert np.all(within_dot_bound(host_bits(bb.dh)[rows], exact, mag))
    # SwiGLU backward rows on the GPU's own dh and gu
    g_gu = host_bits(gu_keep)[rows]
    dgu_ref, _ = O.swiglu_bwd(host_bits(bb.dh)[rows], g_gu)
    assert ulp_diff(host_bits(bb.dgu)[rows], dgu_ref).max() <= 2
    # dW_d and dW_gu on sampled entries: sum_n over all N tokens
    qh = host_u8(pb.qh).reshape(N, H)
    cols_c = rng.integers(0, C, 8)
    cols_h = rng.integers(0, H, 8)
    s_dw = float(np.float32(host_f32(bb.s_dout)[0] * host_f32(pb.s_h)[0]))
    a = gdec(qdout[:, cols_c])                     # [N, 8]
    b = K.e4m3_decode(qh[:, cols_h])               # [N, 8]
    exact = a.T @ b * s_dw
    mag = np.abs(a).T @ np.abs(b) * abs(s_dw)
    got = host_bits(bb.dw_d)[np.ix_(cols_c, cols_h)]
    assert np.all(within_dot_bound(got, exact, mag))
    qdgu = host_u8(bb.qdgu).reshape(N, 2 * H)
    qy = host_u8(pb.qy).reshape(N, C)
    cols_o = rng.integers(0, 2 * H, 8)
    s_gu = float(np.float32(host_f32(bb.s_dgu)[0] * host_f32(pb.s_y)[0]))
    a = gdec(qdgu[:, cols_o])
    b = K.e4m3_decode(qy[:, cols_c])
    exact = a.T @ b * s_gu
    mag = np.abs(a).T @ np.abs(b) * abs(s_gu)
    got = host_bits(bb.dw_gu)[np.ix_(cols_o, cols_c)]
    assert np.all(within_dot_bound(got, exact, mag))
    # dy rows and the RMSNorm backward rows
    wgu = host_u8(pb.w_gu).reshape(2 * H, C)
    s_dy = float(np.float32(host_f32(bb.s_dgu)[0] * host_f32(pb.s_gu)[0]))
    dq = gdec(qdgu[rows])
    wdec = K.e4m3_decode(wgu)
    exact = dq @ wdec * s_dy
    mag = np.abs(dq) @ np.abs(wdec) * abs(s_dy)
    assert np.all(within_dot_bound(host_bits(bb.dy)[rows], exact, mag))
    g_dy, g_r, g_rstd = host_bits(bb.dy)[rows], host_bits(pb.r)[rows], host_f32(pb.rstd)[rows]
    dres_ref, _, _ = O.rmsnorm_bwd(d_out[rows], g_dy, g_r, d["w_norm"], g_rstd)
    assert rms_bwd_close(host_bits(bb.d_res)[rows], dres_ref, d_out[rows], g_dy, g_r, d["w_norm"], g_rstd)


@pytest.mark.parametrize("fp8,grad,conc,zo,tl", [(False, "e4m3", False, False, False),
                                                 (True, "e4m3", False, False, False),
                                                 (True, "e5m2", False, False, False),
                                                 (True, "e4m3", True, False, False),
                                                 (True, "e4m3", False, True, False),
                                                 (True, "e4m3", False, True, True),
                                                 (True, "e5m2", True, False, True)])
def test_block_backward_replays_from_a_hip_graph(F, fp8, grad, conc, zo, tl):
    """Forward + backward (gradients zeroed first) captured once, replayed
    three times with eager work between, equals the eager result bit for bit;
    conc: the two-stream schedule, its second stream forked and joined inside
    the capture; zo: the zero-once abs-max form (its words cleared by the
    captured kernels themselves); tl: tiled operands."""
    say(f"block backward graph replay fp8={fp8} grad={grad} concurrent={conc} zero_once={zo} tiled={tl}")
    from transformer_ffn_block_residual_amd import block
    N, C, H = 200, 384, 256
    d = W.block_inputs(N, C, H, seed=41, w_std=0.1)
    pb = block.PrefillBlock(N, C, H, 1e-5, fp8)
    pb.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    bb = block.BackwardBlock(pb, in_place=False, grad_dtype=grad, concurrent=conc, zero_once=zo, tiled=tl)
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    d_out = dev_bf16(rand_bits((N, C), 1.0, 42))

    def run():
        bb.zero_grads()
        bb.forward(inp, add)
        bb.backward(d_out)

    run()
    torch.cuda.synchronize()
    names = ["d_res", "dw_d", "dw_gu", "dw_norm", "dgu", "dy"]   # dh: not written by the fused form
    if fp8:
        names += ["s_dgu", "am_dres"]
    eager = {n: getattr(bb, n).clone() for n in names}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        run()
    other = empty_bf16(N, 2 * H)
    for rep in range(3):
        for n in names:
            getattr(bb, n).fill_(3.0)
        F.ffn_swiglu_bwd(other, None, bb.dh, bb.gu, N, H)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(bb, n), eager[n]), (rep, n)
