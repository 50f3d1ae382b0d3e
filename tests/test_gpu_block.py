"""GPU parity of the whole FFN block and of the decode FFN against the oracle.

Small workloads are compared element by element end to end.  The full-size
workloads are compared on sampled rows, stage by stage, each stage fed the
GPU's own upstream outputs (codes and scales given the same input are unique,
so they are compared bit for bit), plus an end-to-end check of the sampled rows
through the whole oracle chain conditioned on the GPU's per-tensor abs-maxes.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import codecs as K
from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import (say, dev_bf16, dev_u8, dev_f32, host_bits, host_u8, host_f32, empty_bf16, empty_f32,
                            empty_u8, rel_err, ulp_diff, normwise_err)

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

TOL_BF16, TOL_FP8 = 2e-2, 3e-2


def e2e_err(got, ref, fp8):
    """bf16 path: elementwise relative error (RMS floor).  FP8 path, when the
    oracle takes its own quantisation decisions: error against the tensor's
    abs-max, the scale of the per-tensor e4m3 grid (a code that flips between
    the two chains moves an element by a grid step, not by a fraction of it)."""
    return normwise_err(got, ref) if fp8 else rel_err(got, ref)


@pytest.fixture(scope="module")
def blk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_ffn_block_residual_amd import block
    return block


def _run_block(blk, d, N, C, H, eps, fp8):
    b = blk.PrefillBlock(N, C, H, eps, fp8)
    b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    out = b.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
    # closing residual of this block = the next block's fused residual RMSNorm
    nxt_r, nxt_y, nxt_rstd = empty_bf16(N, C), empty_bf16(N, C), empty_f32(N)
    from transformer_ffn_block_residual_amd import binding as B
    B.ffn_rmsnorm_fwd(nxt_y, nxt_rstd, nxt_r, None, b.r, out, b.w_norm, eps, N, C)
    torch.cuda.synchronize()
    return b, nxt_r


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("N,C,H,outl", [(64, 256, 768, False), (300, 512, 384, True), (1, 128, 128, False)])
def test_block_end_to_end_small(blk, fp8, N, C, H, outl):
    say(f"block e2e fp8={fp8} N={N} C={C} H={H}")
    d = W.block_inputs(N, C, H, seed=1001 if N == 64 else N + C, w_std=0.0, outliers=outl)
    b, nxt_r = _run_block(blk, d, N, C, H, 1e-5, fp8)
    ref = O.block_forward(d["inp"], d["addend"], d["w_norm"], d["w_gu"], d["w_d"], 1e-5, fp8=fp8)
    tol = TOL_FP8 if fp8 else TOL_BF16
    assert np.array_equal(host_bits(b.r), ref["residual"])
    assert rel_err(host_bits(b.y), ref["y"]) < TOL_BF16
    assert e2e_err(host_bits(b.h), ref["h"], fp8) < tol
    assert e2e_err(host_bits(b.out), ref["down"], fp8) < tol
    assert e2e_err(host_bits(nxt_r), ref["next_residual"], fp8) < tol
    if fp8:
        # weights quantised on the GPU are the oracle's codes exactly
        assert np.array_equal(host_u8(b.w_gu), ref["qw_gu"]) and host_f32(b.s_gu)[0] == ref["s_gu"]
        assert np.array_equal(host_u8(b.w_d), ref["qw_d"]) and host_f32(b.s_d)[0] == ref["s_d"]
        # activations: codes given the GPU's own y / h and abs-max are unique
        qy, sy, _ = O.quant_absmax(host_bits(b.y), host_f32(b.am_y)[0])
        assert np.array_equal(host_u8(b.qy), qy) and host_f32(b.s_y)[0] == sy
        qh, sh, _ = O.quant_absmax(host_bits(b.h), host_f32(b.am_h)[0])
        assert np.array_equal(host_u8(b.qh), qh) and host_f32(b.s_h)[0] == sh
        # each stage fed the GPU's own upstream tensors: elementwise tolerance
        h_c, _ = O.swiglu(O.gemm_fp8(host_u8(b.qy), host_f32(b.s_y)[0], ref["qw_gu"], ref["s_gu"]))
        assert rel_err(host_bits(b.h), h_c) < TOL_FP8
        d_c = O.gemm_fp8(host_u8(b.qh), host_f32(b.s_h)[0], ref["qw_d"], ref["s_d"])
        assert rel_err(host_bits(b.out), d_c) < TOL_FP8


@pytest.mark.parametrize("fp8", [False, True])
def test_block_and_decode_replay_from_a_hip_graph(blk, fp8):
    # a captured block forward (and a captured decode) replays to the eager
    # result, bit for bit, on every replay, with eager work and
    # synchronisations between the replays
    N, C, H = 300, 512, 384
    say(f"graph replay fp8={fp8}")
    d = W.block_inputs(N, C, H, seed=77, w_std=0.0)
    b = blk.PrefillBlock(N, C, H, 1e-5, fp8)
    b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    M = 3
    db = blk.DecodeBlock(M, C, H)
    dd = W.decode_inputs(M, C, H, seed=78, with_weights=True)
    db.load_master_weights(dd["w_gate"], dd["w_up"], dd["w_down"])
    xd = dev_bf16(dd["x"])
    b.forward(inp, add)
    db.forward(xd, M)
    torch.cuda.synchronize()
    names = ["r", "y", "rstd", "am_y", "h", "am_h", "out"] + (["qy", "s_y", "qh", "s_h"] if fp8 else [])
    eager = {n: getattr(b, n).clone() for n in names}
    eager_dec = (db.out.clone(), db.h.clone())
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        b.forward(inp, add)
        db.forward(xd, M)
    scratch_y, scratch_rstd = empty_bf16(N, C), empty_f32(N)
    from transformer_ffn_block_residual_amd import binding as B
    for rep in range(3):
        for n in names:
            getattr(b, n).zero_()
        db.out.zero_()
        db.h.zero_()
        B.ffn_rmsnorm_fwd(scratch_y, scratch_rstd, None, None, inp, None, b.w_norm, 1e-5, N, C)  # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(b, n), eager[n]), (rep, n)
        assert torch.equal(db.out, eager_dec[0]) and torch.equal(db.h, eager_dec[1]), rep


def test_block_deterministic(blk):
    N, C, H = 300, 512, 384
    say("block determinism")
    d = W.block_inputs(N, C, H, seed=77)
    b = blk.PrefillBlock(N, C, H, 1e-5, True)
    b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    o1 = b.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"])).clone()
    o2 = b.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"])).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def _sample_rows(N):
    rows = {0, 1, 255, 256, 257, N // 2, N - 257, N - 256, N - 2, N - 1}
    rows |= set(np.random.default_rng(N).integers(0, N, 22).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["prefill", "prefill8", "qwen7b8"])
def test_block_full_size_sampled(blk, name):
    w = W.WORKLOADS[name]
    N, C, H = w.N, w.C, w.H
    say(f"full-size block {name} N={N} C={C} H={H} fp8={w.fp8}")
    d = W.block_inputs(N, C, H, w.seed, w.w_std, w.outliers)
    b = blk.PrefillBlock(N, C, H, w.eps, w.fp8)
    b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    b.forward(dev_bf16(d["inp"]), dev_bf16(d["addend"]))
    torch.cuda.synchronize()
    say(f"full-size block {name}: GPU done, checking on the CPU")
    rows = _sample_rows(N)
    # A1: every row (cheap)
    r_ref, y_ref, rstd_ref, am_y_ref = O.rmsnorm_fwd(d["inp"], d["addend"], d["w_norm"], w.eps)
    gy = host_bits(b.y)
    assert np.array_equal(host_bits(b.r), r_ref)
    assert rel_err(gy, y_ref) < TOL_BF16
    assert np.max(np.abs(host_f32(b.rstd) / rstd_ref - 1)) < 1e-5
    am_y = host_f32(b.am_y)[0]
    assert am_y == np.max(np.abs(K.bf16_bits_to_f64(gy)))
    gh = host_bits(b.h)
    am_h = host_f32(b.am_h)[0]
    assert am_h == np.max(np.abs(K.bf16_bits_to_f64(gh)))
    w_gu, w_d = d["w_gu"], d["w_d"]
    if w.fp8:
        say(f"{name}: oracle weight quantisation")
        qw_gu, s_gu, _ = O.quant_absmax(w_gu)
        qw_d, s_d, _ = O.quant_absmax(w_d)
        say(f"{name}: stage checks")
        assert np.array_equal(host_u8(b.w_gu), qw_gu) and host_f32(b.s_gu)[0] == s_gu
        assert np.array_equal(host_u8(b.w_d), qw_d) and host_f32(b.s_d)[0] == s_d
        # A3: codes of the sampled rows given the GPU's y and abs-max
        qy_all = host_u8(b.qy)
        qy_ref, sy, _ = O.quant_absmax(gy[rows], am_y)
        assert np.array_equal(qy_all[rows], qy_ref) and host_f32(b.s_y)[0] == sy
        # A4+A5 on the sampled rows, from the GPU's codes
        h_cond, _ = O.swiglu(O.gemm_fp8(qy_all[rows], sy, qw_gu, s_gu))
        assert rel_err(gh[rows], h_cond) < TOL_FP8
        # A6
        qh_all = host_u8(b.qh)
        qh_ref, sh, _ = O.quant_absmax(gh[rows], am_h)
        assert np.array_equal(qh_all[rows], qh_ref) and host_f32(b.s_h)[0] == sh
        # A7 from the GPU's codes
        d_cond = O.gemm_fp8(qh_all[rows], sh, qw_d, s_d)
        assert rel_err(host_bits(b.out)[rows], d_cond) < TOL_FP8
        # end to end on the sampled rows, oracle all the way, conditioned only
        # on the per-tensor abs-maxes (global reductions over every row)
        qy_o, sy_o, _ = O.quant_absmax(y_ref[rows], am_y_ref)
        h_o, _ = O.swiglu(O.gemm_fp8(qy_o, sy_o, qw_gu, s_gu))
        qh_o, sh_o, _ = O.quant_absmax(h_o, am_h)
        d_o = O.gemm_fp8(qh_o, sh_o, qw_d, s_d)
        assert normwise_err(host_bits(b.out)[rows], d_o) < TOL_FP8
    else:
        h_cond, _ = O.swiglu(O.gemm_bf16(gy[rows], w_gu))
        assert rel_err(gh[rows], h_cond) < TOL_BF16
        d_cond = O.gemm_bf16(gh[rows], w_d)
        assert rel_err(host_bits(b.out)[rows], d_cond) < TOL_BF16
        h_o, _ = O.swiglu(O.gemm_bf16(y_ref[rows], w_gu))
        d_o = O.gemm_bf16(h_o, w_d)
        assert rel_err(host_bits(b.out)[rows], d_o) < TOL_BF16


@pytest.mark.timeout(300)
def test_decode_full_size_single_token(blk):
    w = W.WORKLOADS["decode"]
    M, C, H = 1, w.C, w.H
    say(f"full-size decode M={M} C={C} H={H}")
    d = W.decode_inputs(M, C, H, w.seed, w.w_std)
    db = blk.DecodeBlock(M, C, H)
    db.load_master_weights(d["w_gate"], d["w_up"], d["w_down"])
    db.forward(dev_bf16(d["x"]))
    torch.cuda.synchronize()
    say("full-size decode: GPU done, checking on the CPU")
    qg, sg = O.quant_rows(d["w_gate"])
    qu, su = O.quant_rows(d["w_up"])
    qd, sd = O.quant_rows(d["w_down"])
    assert np.array_equal(host_u8(db.wg), qg) and np.array_equal(host_f32(db.sg), sg)
    assert np.array_equal(host_u8(db.wu), qu) and np.array_equal(host_f32(db.su), su)
    assert np.array_equal(host_u8(db.wd), qd) and np.array_equal(host_f32(db.sd), sd)
    y_ref, h_ref = O.decode_gemv(d["x"], qg, sg, qu, su, qd, sd)
    gh, gy = host_bits(db.h)[:M], host_bits(db.out)[:M]
    assert rel_err(gh, h_ref) < TOL_BF16
    assert rel_err(gy, O.decode_down(gh, qd, sd)) < TOL_BF16
    assert rel_err(gy, y_ref) < TOL_FP8


@pytest.mark.timeout(300)
def test_decode_batch16_with_prefill_weights(blk):
    # the 16-token decode of the Qwen2-7B-shaped workload runs on the prefill's
    # per-tensor FP8 codes, the scale replicated over the rows
    w = W.WORKLOADS["qwen7b8"]
    M, C, H = w.decode_M, w.C, w.H
    say(f"full-size decode M={M} C={C} H={H} on per-tensor codes")
    d = W.block_inputs(8, C, H, w.seed, w.w_std)   # same weight streams as the prefill
    x = W.decode_inputs(M, C, H, w.seed, with_weights=False)["x"]
    b = blk.PrefillBlock(8, C, H, w.eps, True)
    b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    db = blk.DecodeBlock(M, C, H)
    sg = b.s_gu.expand(H).contiguous()
    sdn = b.s_d.expand(C).contiguous()
    db.set_fp8_weights(b.w_gu[:H], sg, b.w_gu[H:], sg, b.w_d, sdn)
    db.forward(dev_bf16(x))
    torch.cuda.synchronize()
    say("decode M=16: GPU done, checking on the CPU")
    qw_gu, s_gu, _ = O.quant_absmax(d["w_gu"])
    qw_d, s_d, _ = O.quant_absmax(d["w_d"])
    sgv = np.full(H, s_gu, np.float32)
    sdv = np.full(C, s_d, np.float32)
    y_ref, h_ref = O.decode_gemv(x, qw_gu[:H], sgv, qw_gu[H:], sgv, qw_d, sdv)
    gh, gy = host_bits(db.h)[:M], host_bits(db.out)[:M]
    assert rel_err(gh, h_ref) < TOL_BF16
    assert rel_err(gy, O.decode_down(gh, qw_d, sdv)) < TOL_BF16
    assert rel_err(gy, y_ref) < TOL_FP8
