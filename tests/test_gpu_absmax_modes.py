"""GPU tests of the accumulate-into-a-zeroed-word abs-max convention.

``ffn_rmsnorm_fwd_acc`` and ``ffn_gateup_acc`` fold their output's abs-max
into a word the caller zeroed, and ``ffn_quant_absmax_clear`` reads one word
and zeroes another.  ``PrefillBlock.forward_zero_once`` chains them so that no
launch exists only to clear a word.  The results must equal those of the
overwriting calls bit for bit: the abs-max is a max, so folding into a zero
word gives the same value as overwriting, and everything downstream is the
same arithmetic on the same values.
"""

import numpy as np
import pytest
import torch

from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import say, dev_bf16, host_f32, empty_bf16, empty_f32, empty_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_ffn_block_residual_amd import binding, block
    return binding, block


NAMES = ["r", "y", "rstd", "h", "am_h", "out"]
NAMES_FP8 = ["qy", "s_y", "qh", "s_h"]


def _pair(block, d, N, C, H, fp8):
    a = block.PrefillBlock(N, C, H, 1e-5, fp8)
    b = block.PrefillBlock(N, C, H, 1e-5, fp8)
    a.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    b.w_norm, b.w_gu, b.w_d, b.s_gu, b.s_d = a.w_norm, a.w_gu, a.w_d, a.s_gu, a.s_d
    return a, b


@pytest.mark.parametrize("fp8", [True, False])
def test_zero_once_chain_equals_overwriting_chain(mods, fp8):
    """Two calls in a row, the second on inputs a quarter the size, so a
    stale abs-max left from the first call would change its scales."""
    B, block = mods
    N, C, H = 300, 512, 384
    d = W.block_inputs(N, C, H, seed=91, w_std=0.0)
    a, b = _pair(block, d, N, C, H, fp8)
    names = NAMES + (NAMES_FP8 if fp8 else [])
    if not fp8:
        names.remove("am_h")      # the bf16 zero-once chain takes no abs-max
    for call, scale in enumerate((1.0, 0.25)):
        inp = dev_bf16(d["inp"]) * scale
        add = dev_bf16(d["addend"]) * scale
        say(f"zero-once chain fp8={fp8} call {call}")
        a.forward(inp, add)
        b.forward_zero_once(inp, add)
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(a, n), getattr(b, n)), (call, n)
        if fp8:
            assert float(b.am_y.item()) == 0.0                       # cleared for the next call
            assert float(b.am_h.item()) == float(a.am_h.item())
            assert float(a.am_h.item()) > 0.0


def test_zero_once_chain_replays_from_a_hip_graph(mods):
    """The chain holds no clearing launch and no memset, so a captured graph
    replays it unchanged; every replay equals the eager result bit for bit."""
    B, block = mods
    N, C, H = 300, 512, 384
    d = W.block_inputs(N, C, H, seed=92, w_std=0.0)
    a, b = _pair(block, d, N, C, H, True)
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    say("zero-once chain graph capture")
    a.forward(inp, add)
    torch.cuda.synchronize()
    names = NAMES + NAMES_FP8
    eager = {n: getattr(a, n).clone() for n in names}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        b.forward_zero_once(inp, add)
    scratch_y, scratch_rstd = empty_bf16(N, C), empty_f32(N)
    for rep in range(3):
        for n in names:
            getattr(b, n).zero_()
        B.ffn_rmsnorm_fwd(scratch_y, scratch_rstd, None, None, inp, None, b.w_norm, 1e-5, N, C)  # eager work
        torch.cuda.synchronize()
        say(f"zero-once graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(b, n), eager[n]), (rep, n)
        assert float(b.am_y.item()) == 0.0


def test_accumulating_forms_keep_a_larger_word(mods):
    """_acc folds into the word: a preset larger than the output's abs-max
    survives, a smaller one is replaced by the abs-max."""
    B, block = mods
    N, C, H = 64, 256, 256
    d = W.block_inputs(N, C, H, seed=93, w_std=0.0)
    inp = dev_bf16(d["inp"])
    w_norm = dev_bf16(d["w_norm"])
    y, rstd, am_ref = empty_bf16(N, C), empty_f32(N), empty_f32(1)
    say("rmsnorm abs-max reference")
    B.ffn_rmsnorm_fwd(y, rstd, None, am_ref, inp, None, w_norm, 1e-5, N, C)
    torch.cuda.synchronize()
    ref = float(am_ref.item())
    assert ref == float(y.float().abs().max().item())
    for preset, want in ((1e6, 1e6), (ref * 0.5, ref), (0.0, ref)):
        y2, rstd2 = empty_bf16(N, C), empty_f32(N)
        am = torch.full((1,), preset, dtype=torch.float32, device="cuda")
        say(f"rmsnorm_fwd_acc preset={preset}")
        B.ffn_rmsnorm_fwd_acc(y2, rstd2, None, am, inp, None, w_norm, 1e-5, N, C)
        torch.cuda.synchronize()
        assert torch.equal(y2, y) and torch.equal(rstd2, rstd)
        assert float(am.item()) == np.float32(want)
    # gate+up: bf16 product, abs-max of h folded in
    w_gu = dev_bf16(d["w_gu"])
    h_ref, amh_ref = empty_bf16(N, H), empty_f32(1)
    say("gateup abs-max reference")
    B.ffn_gateup(h_ref, amh_ref, y, None, w_gu, None, B.FFN_BF16, 1, N, C, H)
    torch.cuda.synchronize()
    href = float(amh_ref.item())
    assert href == float(h_ref.float().abs().max().item())
    for preset, want in ((1e6, 1e6), (href * 0.5, href), (0.0, href)):
        h2 = empty_bf16(N, H)
        am = torch.full((1,), preset, dtype=torch.float32, device="cuda")
        say(f"gateup_acc preset={preset}")
        B.ffn_gateup_acc(h2, am, y, None, w_gu, None, B.FFN_BF16, N, C, H)
        torch.cuda.synchronize()
        assert torch.equal(h2, h_ref)
        assert float(am.item()) == np.float32(want)


def test_quant_clear_equals_quant_and_zeroes_its_word(mods):
    B, block = mods
    n = 64 * 1000 + 13                       # a ragged tail after the 16-element groups
    x = dev_bf16(W.block_inputs(64, 1024, 128, seed=94)["inp"]).reshape(-1)[:n].contiguous()
    q_ref, s_ref, am = empty_u8(n), empty_f32(1), empty_f32(1)
    say("quant reference")
    B.ffn_quant_absmax(q_ref, s_ref, am, x, n, 1)
    torch.cuda.synchronize()
    words = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    words[0] = am[0]
    q, s = empty_u8(n), words[1:2]
    say("quant_absmax_clear")
    B.ffn_quant_absmax_clear(q, s, words[0:1], x, n, words[2:3])
    torch.cuda.synchronize()
    assert torch.equal(q, q_ref)
    assert torch.equal(s, s_ref)
    w = host_f32(words)
    assert w[0] == host_f32(am)[0] and w[2] == 0.0 and w[3] == 7.0
