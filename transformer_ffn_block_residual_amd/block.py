"""The FFN block as a sequence of C-ABI calls on device buffers.

``PrefillBlock`` runs one block forward over N token rows, as the trainer's
``LLamaModel::_forward_block`` runs its FFN half (llmq llama_model.cpp):

  ffn_rmsnorm_fwd   r = inp + addend, y = RMSNorm(r) * w, rstd, max|y|
  ffn_quant_absmax  y -> e4m3 with max|y|                       (FP8 only)
  ffn_gateup        [N,C] x [2H,C]^T, fused SwiGLU epilogue, max|h|
  ffn_quant_absmax  h -> e4m3 with max|h|                       (FP8 only)
  ffn_down          [N,H] x [C,H]^T

``forward_known_h_absmax`` is the FP8 form whose gate+up epilogue quantises h
under an abs-max known beforehand (``ffn_gateup_swiglu_quant``), as the
trainer's recompute pass re-creates its quantised SwiGLU output.

The residual that closes the block (r + down) is the next block's first
``ffn_rmsnorm_fwd`` (``LLamaModel::forward`` fuses it there), so a chain of
blocks feeds ``(r, down)`` of one block into ``(inp, addend)`` of the next.

``DecodeBlock`` holds FP8 weights with per-row scales and runs
``ffn_decode_gemv`` for 1..32 tokens (metrale dense_ffn_decode.rs,
``DenseFfnLayer::forward``, FP8 arm), or one of its other arms
(``ffn_decode_gemv_arm``, 1..4 tokens); ``DecodeBlockBf16`` holds bf16
weights and runs ``ffn_decode_gemv_bf16`` (the bf16 arm, 1..4 tokens).

Buffers are allocated once, at construction, through torch; the calls
themselves allocate nothing.  Every step of the arithmetic runs in libffn.so.
"""

import torch

from . import binding as B


def _bf16_dev(bits_u16):
    """Host uint16 bf16 bit patterns -> device bf16 tensor (a copy)."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def _f32(*shape):
    return torch.empty(*shape, dtype=torch.float32, device="cuda")


def _bf16(*shape):
    return torch.empty(*shape, dtype=torch.bfloat16, device="cuda")


def _u8(*shape):
    return torch.empty(*shape, dtype=torch.uint8, device="cuda")


class PrefillBlock:
    def __init__(self, N, C, H, eps, fp8):
        self.N, self.C, self.H, self.eps, self.fp8 = N, C, H, float(eps), bool(fp8)
        self.r = _bf16(N, C)
        self.y = _bf16(N, C)
        self.rstd = _f32(N)
        self.am_y = _f32(1)
        self.h = _bf16(N, H)
        self.am_h = _f32(1)
        self.out = _bf16(N, C)
        if self.fp8:
            self.qy, self.s_y = _u8(N, C), _f32(1)
            self.qh, self.s_h = _u8(N, H), _f32(1)

    def load_weights(self, w_norm, w_gu, w_d):
        """Device bf16 weights (tensors or host bit-pattern arrays).  For FP8 the
        projections are quantised here, per tensor, with their own abs-max."""
        as_dev = (lambda w: w if isinstance(w, torch.Tensor) else _bf16_dev(w))
        self.w_norm = as_dev(w_norm)
        w_gu, w_d = as_dev(w_gu), as_dev(w_d)
        C, H = self.C, self.H
        if not self.fp8:
            self.w_gu, self.w_d = w_gu, w_d
            self.s_gu = self.s_d = None
            return
        self.w_gu, self.s_gu, am = _u8(2 * H, C), _f32(1), _f32(1)
        B.ffn_quant_absmax(self.w_gu, self.s_gu, am, w_gu, 2 * H * C, 1)
        self.w_d, self.s_d, am2 = _u8(C, H), _f32(1), _f32(1)
        B.ffn_quant_absmax(self.w_d, self.s_d, am2, w_d, C * H, 1)
        torch.cuda.current_stream().synchronize()

    def forward(self, inp, addend, stream=None):
        """One block forward; returns the down-projection output [N, C] (the
        tensor the next block adds to ``self.r``)."""
        N, C, H = self.N, self.C, self.H
        B.ffn_rmsnorm_fwd(self.y, self.rstd, self.r if addend is not None else None, self.am_y,
                          inp, addend, self.w_norm, self.eps, N, C, stream)
        if self.fp8:
            B.ffn_quant_absmax(self.qy, self.s_y, self.am_y, self.y, N * C, 0, stream)
            B.ffn_gateup(self.h, self.am_h, self.qy, self.s_y, self.w_gu, self.s_gu, B.FFN_E4M3, 1, N, C, H,
                         stream)
            B.ffn_quant_absmax(self.qh, self.s_h, self.am_h, self.h, N * H, 0, stream)
            B.ffn_down(self.out, self.qh, self.s_h, self.w_d, self.s_d, B.FFN_E4M3, N, H, C, stream)
        else:
            B.ffn_gateup(self.h, self.am_h, self.y, None, self.w_gu, None, B.FFN_BF16, 1, N, C, H, stream)
            B.ffn_down(self.out, self.h, None, self.w_d, None, B.FFN_BF16, N, H, C, stream)
        return self.out

    def forward_known_h_absmax(self, inp, addend, h_absmax_known, h_absmax_out, stream=None):
        """FP8 block forward whose h is quantised in the gate+up epilogue with
        an abs-max known beforehand (the recompute form: llmq llama_model.cpp,
        ``LLamaModel::_recompute_block``, ``swiglu_forward_quant``): no bf16 h
        and no separate quantisation pass.  ``h_absmax_out`` receives this
        call's abs-max of h (the next call's known value; it must be another
        buffer than ``h_absmax_known``)."""
        assert self.fp8, "the known-abs-max form is an FP8 path"
        N, C, H = self.N, self.C, self.H
        B.ffn_rmsnorm_fwd(self.y, self.rstd, self.r if addend is not None else None, self.am_y,
                          inp, addend, self.w_norm, self.eps, N, C, stream)
        B.ffn_quant_absmax(self.qy, self.s_y, self.am_y, self.y, N * C, 0, stream)
        B.ffn_gateup_swiglu_quant(self.qh, self.s_h, h_absmax_out, h_absmax_known, self.qy, self.s_y, self.w_gu,
                                  self.s_gu, B.FFN_E4M3, N, C, H, stream)
        B.ffn_down(self.out, self.qh, self.s_h, self.w_d, self.s_d, B.FFN_E4M3, N, H, C, stream)
        return self.out


class DecodeBlock:
    def __init__(self, M, C, H):
        self.M, self.C, self.H = M, C, H
        self.h = _bf16(max(M, 1), H)
        self.out = _bf16(max(M, 1), C)

    def load_master_weights(self, w_gate, w_up, w_down):
        """bf16 master weights -> e4m3 codes with per-row scales (ffn_quant_rows)."""
        as_dev = (lambda w: w if isinstance(w, torch.Tensor) else _bf16_dev(w))
        C, H = self.C, self.H
        self.wg, self.sg = _u8(H, C), _f32(H)
        self.wu, self.su = _u8(H, C), _f32(H)
        self.wd, self.sd = _u8(C, H), _f32(C)
        B.ffn_quant_rows(self.wg, self.sg, as_dev(w_gate), H, C)
        B.ffn_quant_rows(self.wu, self.su, as_dev(w_up), H, C)
        B.ffn_quant_rows(self.wd, self.sd, as_dev(w_down), C, H)
        torch.cuda.current_stream().synchronize()

    def set_fp8_weights(self, wg, sg, wu, su, wd, sd):
        """Use existing e4m3 codes and per-row scales (device tensors)."""
        self.wg, self.sg, self.wu, self.su, self.wd, self.sd = wg, sg, wu, su, wd, sd

    def forward(self, x, M=None, stream=None):
        M = self.M if M is None else M
        B.ffn_decode_gemv(self.out, self.h, x, self.wg, self.sg, self.wu, self.su, self.wd, self.sd,
                          M, self.C, self.H, stream)
        return self.out

    def _gu(self):
        if not hasattr(self, "gu"):
            self.gu = _bf16(max(self.M, 1), 2 * self.H)   # g | u workspace of the non-split arms
        return self.gu

    def forward_arm(self, x, arm, M=None, stream=None):
        M = self.M if M is None else M
        B.ffn_decode_gemv_arm(self.out, self.h, self._gu(), x, self.wg, self.sg, self.wu, self.su, self.wd,
                              self.sd, arm, M, self.C, self.H, stream)
        return self.out

    def bind(self, x, M=None, stream=None, arm=None):
        """A no-argument callable that runs forward(x, M, stream) (or
        forward_arm with ``arm``) with the argument checks done once (for
        per-token loops)."""
        M = self.M if M is None else M
        if arm is None:
            return B.bind_decode_gemv(self.out, self.h, x, self.wg, self.sg, self.wu, self.su, self.wd, self.sd,
                                      M, self.C, self.H, stream)
        return B.bind_decode_gemv_arm(self.out, self.h, self._gu(), x, self.wg, self.sg, self.wu, self.su,
                                      self.wd, self.sd, arm, M, self.C, self.H, stream)


class DecodeBlockBf16:
    def __init__(self, M, C, H):
        self.M, self.C, self.H = M, C, H
        self.h = _bf16(max(M, 1), H)
        self.out = _bf16(max(M, 1), C)

    def load_weights(self, w_gate, w_up, w_down):
        """bf16 weights: device tensors (kept as given) or host bit patterns (copied)."""
        as_dev = (lambda w: w if isinstance(w, torch.Tensor) else _bf16_dev(w))
        self.wg, self.wu, self.wd = as_dev(w_gate), as_dev(w_up), as_dev(w_down)

    def forward(self, x, M=None, stream=None):
        M = self.M if M is None else M
        B.ffn_decode_gemv_bf16(self.out, self.h, x, self.wg, self.wu, self.wd, M, self.C, self.H, stream)
        return self.out

    def bind(self, x, M=None, stream=None):
        M = self.M if M is None else M
        return B.bind_decode_gemv_bf16(self.out, self.h, x, self.wg, self.wu, self.wd, M, self.C, self.H, stream)
