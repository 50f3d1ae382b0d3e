"""ffn_decode_gemv_packed_noalloc (the packed decode with the library's
built-in device scratch as its workspace) against ffn_decode_gemv_packed with
a caller workspace, through the C ABI: equal bit for bit, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents, which must not leak into the second)."""

import numpy as np
import pytest
import torch

import oracle as O
from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import say, dev_bf16, dev_u8, empty_bf16, empty_u8, host_bits, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_ffn_block_residual_amd as F
    return F


def _packed_weights(F, d):
    out = {}
    for k in ("w_gate", "w_up", "w_down"):
        rows, cols = d[k].shape
        q, s = O.quant_rows(d[k])
        p = empty_u8(rows, cols)
        F.ffn_decode_pack_weight(p, dev_u8(q), rows, cols)
        out[k] = (p, torch.from_numpy(s).cuda(), q, s)
    return out


def test_noalloc_decode_equals_the_workspace_form_on_two_calls(F):
    assert F.ffn_decode_noalloc_scratch_bytes() == 8 << 20
    C, H = 3584, 18944          # the Qwen2-7B shape: the largest workspace of the workloads
    cases = [(16, C, H), (5, C, H), (1, 1024, 2048)]
    for M, C_, H_ in cases:
        say(f"no-alloc decode M={M} C={C_} H={H_}")
        assert F.ffn_decode_packed_workspace_bytes(M, C_, H_) <= F.ffn_decode_noalloc_scratch_bytes()
        d = W.decode_inputs(M, C_, H_, seed=M + C_ + H_)
        pw = _packed_weights(F, d)
        args = (dev_bf16(d["x"]), pw["w_gate"][0], pw["w_gate"][1], pw["w_up"][0], pw["w_up"][1],
                pw["w_down"][0], pw["w_down"][1], M, C_, H_)
        out_a, h_a = empty_bf16(M, C_).fill_(3.0), empty_bf16(M, H_).fill_(3.0)
        F.ffn_decode_gemv_packed_noalloc(out_a, h_a, *args)
        ws = empty_bf16(F.ffn_decode_packed_workspace_bytes(M, C_, H_) // 2).fill_(-7.0)
        out_b, h_b = empty_bf16(M, C_), empty_bf16(M, H_)
        F.ffn_decode_gemv_packed(out_b, h_b, ws, *args)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b) and torch.equal(h_a, h_b)
        # and the oracle, to the packed decode's tolerance
        y_ref, _ = O.decode_gemv(d["x"], pw["w_gate"][2], pw["w_gate"][3], pw["w_up"][2], pw["w_up"][3],
                                 pw["w_down"][2], pw["w_down"][3])
        assert rel_err(host_bits(out_a), y_ref) < 3e-2


def test_noalloc_decode_rejects_sizes_beyond_the_scratch(F):
    M, C, H = 16, 131072, 128   # 12.6 MB of workspace, small weights
    assert F.ffn_decode_packed_workspace_bytes(M, C, H) > F.ffn_decode_noalloc_scratch_bytes()
    with pytest.raises(F.FFNError, match="scratch"):
        F.ffn_decode_gemv_packed_noalloc(empty_bf16(M, C), empty_bf16(M, H), empty_bf16(M, C),
                                         empty_u8(H, C), torch.empty(H, device="cuda"),
                                         empty_u8(H, C), torch.empty(H, device="cuda"),
                                         empty_u8(C, H), torch.empty(C, device="cuda"), M, C, H)
