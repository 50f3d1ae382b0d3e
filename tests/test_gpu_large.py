"""Operands past 2 and 4 GiB: the kernels' 64-bit addressing, checked on whole
tensors.  (A GEMM input operand may reach 4 GiB, its output and the row-wise
kernels' operands may exceed it.)

Each input repeats a seeded block of P rows (P = 4099, prime, so that a byte
offset that wrapped at 2^31 or 2^32 would land on a different row of the block
and change the result).  The oracle computes the block once; the expected
tensor is that result repeated, compared with the GPU's whole output on the
device.  Integer-valued e4m3 operands make the GEMM sums exact (unique
results, bit-exact); the residual sum, the e4m3 codes and the abs-maxes are
unique too.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import codecs as K
from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import (say, dev_bf16, dev_u8, dev_f32, host_bits, host_f32, empty_bf16, empty_f32,
                            empty_u8, ulp_diff)

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

P = 4099
GIB4 = 1 << 32


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_ffn_block_residual_amd as F
    yield F
    torch.cuda.empty_cache()


def _repeat_rows(block, n):
    """The device block [P, ...] repeated along rows to n rows."""
    reps = (n + block.shape[0] - 1) // block.shape[0]
    return block.repeat(reps, *([1] * (block.dim() - 1)))[:n].contiguous()


def _int_e4m3(shape, seed):
    # codes of the integers -4..4, exact in e4m3: every partial sum is an exact integer
    vals = np.random.default_rng(seed).integers(-4, 5, shape).astype(np.float32)
    return K.e4m3_encode(vals)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_gateup_token_operand_up_to_4gib(F):
    # x: [N, 1024] e4m3, 300 rows short of 4 GiB (the largest input operand a
    # GEMM takes); rows from 2^21 on start past 2^31 bytes; out 2.1 GB
    C, H = 1024, 128
    N = GIB4 // C - 300
    say(f"gateup e4m3, x up to 4 GiB: N={N} C={C} H={H}")
    qx, qw = _int_e4m3((P, C), 11), _int_e4m3((2 * H, C), 12)
    ref = torch.from_numpy(O.gemm_fp8(qx, np.float32(1), qw, np.float32(1)).view(np.int16)).cuda()
    x = _repeat_rows(dev_u8(qx), N)
    one = dev_f32([1.0])
    out = empty_bf16(N, 2 * H)
    F.ffn_gateup(out, None, x, one, dev_u8(qw), one, F.FFN_E4M3, 0, N, C, H)
    torch.cuda.synchronize()
    del x
    assert torch.equal(out.view(torch.int16), _repeat_rows(ref, N))
    del out
    _free()


def test_down_output_past_4gib(F):
    # out: [N, 1024] bf16 = 4.3 GB; the last 300 token rows are written past 2^32 bytes
    H, C = 128, 1024
    N = GIB4 // (2 * C) + 300
    say(f"down e4m3, out past 4 GiB: N={N} H={H} C={C}")
    qh, qw = _int_e4m3((P, H), 13), _int_e4m3((C, H), 14)
    ref = torch.from_numpy(O.gemm_fp8(qh, np.float32(1), qw, np.float32(1)).view(np.int16)).cuda()
    h = _repeat_rows(dev_u8(qh), N)
    one = dev_f32([1.0])
    out = empty_bf16(N, C)
    F.ffn_down(out, h, one, dev_u8(qw), one, F.FFN_E4M3, N, H, C)
    torch.cuda.synchronize()
    del h
    assert torch.equal(out.view(torch.int16), _repeat_rows(ref, N))
    del out
    _free()


def test_rmsnorm_operands_past_4gib(F):
    # inp, addend, y, residual: [N, 1024] bf16 = 4.3 GB each
    C = 1024
    N = GIB4 // (2 * C) + 77
    say(f"rmsnorm, operands past 4 GiB: N={N} C={C}")
    d = W.block_inputs(P, C, 128, seed=15)
    r_ref, y_ref, rstd_ref, _ = O.rmsnorm_fwd(d["inp"], d["addend"], d["w_norm"], 1e-5)
    inp = _repeat_rows(dev_bf16(d["inp"]), N)
    addend = _repeat_rows(dev_bf16(d["addend"]), N)
    y, rstd, res, am = empty_bf16(N, C), empty_f32(N), empty_bf16(N, C), empty_f32(1)
    F.ffn_rmsnorm_fwd(y, rstd, res, am, inp, addend, dev_bf16(d["w_norm"]), 1e-5, N, C)
    torch.cuda.synchronize()
    del inp, addend
    # the residual sum is unique
    assert torch.equal(res.view(torch.int16), _repeat_rows(dev_bf16(r_ref).view(torch.int16), N))
    del res
    # every row equals its copy in the first block, bit for bit (same row, same
    # arithmetic), and the first block agrees with the oracle as in the
    # small-shape test
    assert torch.equal(y.view(torch.int16), _repeat_rows(y[:P].view(torch.int16), N))
    assert torch.equal(rstd, _repeat_rows(rstd[:P], N))
    g_rstd, gy = host_f32(rstd[:P]), host_bits(y[:P])
    assert np.max(np.abs(g_rstd / rstd_ref - 1)) < 1e-5
    y_cond, _ = O.rms_apply(r_ref, g_rstd, d["w_norm"])
    assert ulp_diff(gy, y_cond).max() <= 1
    assert host_f32(am)[0] == np.max(np.abs(K.bf16_bits_to_f64(gy)))
    del y, rstd
    _free()


def test_quant_absmax_past_2pow32_elements(F):
    # x: 2^32 + 300 * 1024 bf16 elements (8.6 GB), codes 4.3 GB; the element
    # count itself exceeds 32 bits
    C = 1024
    N = GIB4 // C + 300
    n = N * C
    say(f"quant_absmax, {n} elements")
    d = W.block_inputs(P, C, 128, seed=16, outliers=True)
    q_ref, s_ref, am_ref = O.quant_absmax(d["inp"])
    x = _repeat_rows(dev_bf16(d["inp"]), N)
    q, scale, am = empty_u8(N, C), empty_f32(1), empty_f32(1)
    F.ffn_quant_absmax(q, scale, am, x, n, 1)
    torch.cuda.synchronize()
    del x
    assert host_f32(am)[0] == np.float32(am_ref)
    assert host_f32(scale)[0] == np.float32(s_ref)
    assert torch.equal(q, _repeat_rows(dev_u8(q_ref), N))
    del q
    _free()
