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

``BackwardBlock`` runs the FFN half of the trainer's ``_backward_block`` for
a ``PrefillBlock``: a forward that keeps the up-projection output (``MlpUp``,
as the trainer keeps or recomputes it), then ``backward_qmm`` through the down
projection, ``swiglu_backward``, ``backward_qmm`` through the up projection and
``rmsnorm_backward`` (llmq llama_model.cpp, ``LLamaModel::_backward_block``,
``backward_qmm``).  The transposed operands that the TN products need are made
by ``ffn_transpose`` / ``ffn_quant_transpose`` with the token dimension padded
to a multiple of 128 (zeros), the GEMM's K granularity.  The transposed
weights are made once per weight update (``PrefillBlock.weights_version``) and
reused by every backward until the weights change again.

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
    """One FFN block's prefill forward over N tokens.  tiled: the operands of
    both GEMMs (the weights, and y and h, or their e4m3 codes) are kept in
    the library's tiled layout (``ffn_tile_pack``), which the GEMMs read a
    contiguous KiB at a time; the results are those of the row-major operands
    bit for bit.  ``qy`` and ``qh`` (FP8), or ``y`` and ``h`` (bf16), then
    hold tiled data; the tiled block runs ``forward_zero_once`` (and, FP8,
    ``forward_known_h_absmax``)."""

    def __init__(self, N, C, H, eps, fp8, tiled=False):
        self.N, self.C, self.H, self.eps, self.fp8 = N, C, H, float(eps), bool(fp8)
        self.tiled = bool(tiled)
        bf16_tiled = self.tiled and not self.fp8
        self.r = _bf16(N, C)
        self.y = _bf16(B.ffn_tile_bytes(N, 2 * C) // 2) if bf16_tiled else _bf16(N, C)
        self.rstd = _f32(N)
        # the abs-max table, zeroed once here: am_y and am_h in words 0 and 4
        # (16 bytes apart); forward() overwrites them, forward_zero_once()
        # accumulates into them and clears each after its consumer
        self.am_tab = torch.zeros(8, dtype=torch.float32, device="cuda")
        self.am_y = self.am_tab[0:1]
        self.h = _bf16(B.ffn_tile_bytes(N, 2 * H) // 2) if bf16_tiled else _bf16(N, H)
        self.am_h = self.am_tab[4:5]
        self.out = _bf16(N, C)
        if self.fp8:
            if self.tiled:
                self.qy, self.qh = _u8(B.ffn_tile_bytes(N, C)), _u8(B.ffn_tile_bytes(N, H))
            else:
                self.qy, self.qh = _u8(N, C), _u8(N, H)
            self.s_y, self.s_h = _f32(1), _f32(1)
        # bumped whenever the projection weights change; what is derived from
        # them (the backward's transposed weights) is remade when it moves
        self.weights_version = 0

    def weights_changed(self):
        """Declare that the projection weights were updated in place (an
        optimizer step), so that what is derived from them is remade."""
        self.weights_version += 1

    def load_weights(self, w_norm, w_gu, w_d):
        """Device bf16 weights (tensors or host bit-pattern arrays).  For FP8 the
        projections are quantised here, per tensor, with their own abs-max."""
        self.weights_changed()
        as_dev = (lambda w: w if isinstance(w, torch.Tensor) else _bf16_dev(w))
        self.w_norm = as_dev(w_norm)
        w_gu, w_d = as_dev(w_gu), as_dev(w_d)
        C, H = self.C, self.H
        if not self.fp8:
            self.w_gu_rows, self.w_d_rows = w_gu, w_d
            self.w_gu, self.w_d = w_gu, w_d
            self.s_gu = self.s_d = None
            if self.tiled:
                self.w_gu = _bf16(B.ffn_tile_bytes(2 * H, 2 * C) // 2)
                self.w_d = _bf16(B.ffn_tile_bytes(C, 2 * H) // 2)
                B.ffn_tile_pack(self.w_gu.view(torch.uint8), w_gu.view(torch.uint8), 2 * H, 2 * C)
                B.ffn_tile_pack(self.w_d.view(torch.uint8), w_d.view(torch.uint8), C, 2 * H)
                torch.cuda.current_stream().synchronize()
            return
        self.w_gu, self.s_gu, am = _u8(2 * H, C), _f32(1), _f32(1)
        B.ffn_quant_absmax(self.w_gu, self.s_gu, am, w_gu, 2 * H * C, 1)
        self.w_d, self.s_d, am2 = _u8(C, H), _f32(1), _f32(1)
        B.ffn_quant_absmax(self.w_d, self.s_d, am2, w_d, C * H, 1)
        # the row-major codes stay available (the decode reads them)
        self.w_gu_rows, self.w_d_rows = self.w_gu, self.w_d
        if self.tiled:
            self.w_gu, self.w_d = _u8(B.ffn_tile_bytes(2 * H, C)), _u8(B.ffn_tile_bytes(C, H))
            B.ffn_tile_pack(self.w_gu, self.w_gu_rows, 2 * H, C)
            B.ffn_tile_pack(self.w_d, self.w_d_rows, C, H)
        torch.cuda.current_stream().synchronize()

    def forward(self, inp, addend, stream=None):
        """One block forward; returns the down-projection output [N, C] (the
        tensor the next block adds to ``self.r``)."""
        N, C, H = self.N, self.C, self.H
        assert not self.tiled, "the tiled block runs forward_zero_once or forward_known_h_absmax"
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

    def forward_zero_once(self, inp, addend, stream=None):
        """The same forward with the trainer's abs-max convention (llmq
        llama_model.cpp, ``LLamaModel::forward``: the abs-max table is zeroed
        once and every producer accumulates into its slot): the RMSNorm and
        the gate+up epilogue accumulate into the table; the quantiser of y
        clears h's slot and the quantiser of h clears y's slot, so the next
        call finds both zero and no call clears a word with a launch of its
        own.  Results equal forward()'s bit for bit.  Afterwards am_y reads 0
        (cleared for the next call) and am_h holds max|h|.  The bf16 block has
        no quantiser, so it takes no abs-max at all."""
        N, C, H = self.N, self.C, self.H
        r = self.r if addend is not None else None
        if not self.fp8:
            if self.tiled:
                B.ffn_rmsnorm_fwd_tiled(self.y, self.rstd, r, None, inp, addend, self.w_norm, self.eps, N, C, stream)
                B.ffn_gateup_tiled_bf16(self.h, None, self.y, self.w_gu, N, C, H, stream)
                B.ffn_down_tiled_bf16(self.out, self.h, self.w_d, N, H, C, stream)
                return self.out
            B.ffn_rmsnorm_fwd(self.y, self.rstd, r, None, inp, addend, self.w_norm, self.eps, N, C, stream)
            B.ffn_gateup(self.h, None, self.y, None, self.w_gu, None, B.FFN_BF16, 1, N, C, H, stream)
            B.ffn_down(self.out, self.h, None, self.w_d, None, B.FFN_BF16, N, H, C, stream)
            return self.out
        B.ffn_rmsnorm_fwd_acc(self.y, self.rstd, r, self.am_y, inp, addend, self.w_norm, self.eps, N, C, stream)
        if self.tiled:
            B.ffn_quant_absmax_clear_tiled(self.qy, self.s_y, self.am_y, self.y, N, C, self.am_h, stream)
            B.ffn_gateup_acc_tiled(self.h, self.am_h, self.qy, self.s_y, self.w_gu, self.s_gu, N, C, H, stream)
            B.ffn_quant_absmax_clear_tiled(self.qh, self.s_h, self.am_h, self.h, N, H, self.am_y, stream)
            B.ffn_down_tiled(self.out, self.qh, self.s_h, self.w_d, self.s_d, N, H, C, stream)
            return self.out
        B.ffn_quant_absmax_clear(self.qy, self.s_y, self.am_y, self.y, N * C, self.am_h, stream)
        B.ffn_gateup_acc(self.h, self.am_h, self.qy, self.s_y, self.w_gu, self.s_gu, B.FFN_E4M3, N, C, H, stream)
        B.ffn_quant_absmax_clear(self.qh, self.s_h, self.am_h, self.h, N * H, self.am_y, stream)
        B.ffn_down(self.out, self.qh, self.s_h, self.w_d, self.s_d, B.FFN_E4M3, N, H, C, stream)
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
        if self.tiled:
            B.ffn_quant_absmax_clear_tiled(self.qy, self.s_y, self.am_y, self.y, N, C, None, stream)
            B.ffn_gateup_swiglu_quant_tiled(self.qh, self.s_h, h_absmax_out, h_absmax_known, self.qy, self.s_y,
                                            self.w_gu, self.s_gu, N, C, H, stream)
            B.ffn_down_tiled(self.out, self.qh, self.s_h, self.w_d, self.s_d, N, H, C, stream)
            return self.out
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


class DecodeBlockPacked(DecodeBlock):
    """DecodeBlock with its e4m3 weights kept in the packed decode layout
    (ffn_decode_pack_weight) and run through ffn_decode_gemv_packed: the
    faster form from three to 32 tokens.  The row scales are DecodeBlock's; the
    row-major codes are not kept."""

    def __init__(self, M, C, H):
        super().__init__(M, C, H)
        self.ws = _bf16(B.ffn_decode_packed_workspace_bytes(max(M, 1), C, H) // 2)

    def _pack(self, wg, wu, wd):
        C, H = self.C, self.H
        self.wg, self.wu, self.wd = _u8(H, C), _u8(H, C), _u8(C, H)
        B.ffn_decode_pack_weight(self.wg, wg, H, C)
        B.ffn_decode_pack_weight(self.wu, wu, H, C)
        B.ffn_decode_pack_weight(self.wd, wd, C, H)
        torch.cuda.current_stream().synchronize()

    def load_master_weights(self, w_gate, w_up, w_down):
        super().load_master_weights(w_gate, w_up, w_down)
        self._pack(self.wg, self.wu, self.wd)

    def set_fp8_weights(self, wg, sg, wu, su, wd, sd):
        """Pack existing row-major e4m3 codes; keep their per-row scales."""
        self.sg, self.su, self.sd = sg, su, sd
        self._pack(wg, wu, wd)

    def forward(self, x, M=None, stream=None):
        M = self.M if M is None else M
        B.ffn_decode_gemv_packed(self.out, self.h, self.ws, x, self.wg, self.sg, self.wu, self.su, self.wd,
                                 self.sd, M, self.C, self.H, stream)
        return self.out

    def forward_arm(self, x, arm, M=None, stream=None):
        raise NotImplementedError("the packed decode runs the split-SiLU arm only")

    def bind(self, x, M=None, stream=None, arm=None):
        if arm is not None:
            raise NotImplementedError("the packed decode runs the split-SiLU arm only")
        M = self.M if M is None else M
        return B.bind_decode_gemv_packed(self.out, self.h, self.ws, x, self.wg, self.sg, self.wu, self.su,
                                         self.wd, self.sd, M, self.C, self.H, stream)


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


def _round_up(n, m):
    return (n + m - 1) // m * m


class BackwardBlock:
    """Forward (keeping gu) and backward of one FFN block; gradients of the
    three weights accumulate across calls (``zero_grads`` clears them).
    in_place: the SwiGLU backward overwrites gu with its gradient, as the
    trainer does; otherwise it goes to a buffer of its own (``dgu``) and gu
    survives for another backward.  grad_dtype ("e4m3" or "e5m2", FP8 blocks
    only): the format of the quantised gradients (the output gradient and
    dMlpUp), each scaled by its abs-max over that format's largest value;
    weights and activations stay e4m3.  fuse_swiglu_bwd: the down
    projection's data gradient and the SwiGLU backward run as one kernel
    (ffn_matmul_tn_swiglu_bwd), which never writes dh; False runs them as
    ffn_matmul_tn + ffn_swiglu_bwd and keeps dh (same results bit for bit).
    concurrent: each projection's weight gradient (with the transposes only it
    needs) runs on a second stream beside the data gradient, both launched
    with FFN_TN_TILE_GRID, so that the partial last round of tiles of one
    product can fill with tiles of the other; the second stream joins before
    backward returns.  Same results bit for bit; per-phase marks (``mark``)
    take the serial order.  Off by default: at the Qwen2-7B shape it measures
    the same as the serial order (the products are bound by the chip's power,
    not by idle CUs).
    zero_once: the trainer's abs-max convention for the backward's two
    gradient slots (llmq llama_model.cpp, LLamaRunState: DMlpUp.Quant.Stats
    and DResAtt.Quant.Stats in the abs-max table that LLamaModel::forward
    zeroes once): the SwiGLU backward and the RMSNorm backward accumulate
    into zeroed words; the quantiser of dMlpUp clears d_res's word and the
    RMSNorm backward clears dMlpUp's after its consumer has run, so no call
    clears a word with a launch of its own.  Gradients equal the default
    form's bit for bit; afterwards am_dres holds max|d_res| (the upstream
    block's d_out_absmax) and am_dgu reads 0.  A bf16 block has no quantiser
    of these gradients and so takes no abs-max at all.  Chosen at
    construction (the words start at zero then).
    tiled (FP8 only): the four TN products read their operands (gradient,
    weight and activation codes, as transposed or quantised here) in the
    library's tiled layout (FFN_TN_TILED), which the transposing quantisers
    and transposes write directly; gradients equal the row-major form's bit
    for bit."""

    def __init__(self, fwd, in_place=True, grad_dtype="e4m3", fuse_swiglu_bwd=True, concurrent=False,
                 zero_once=False, tiled=False):
        if getattr(fwd, "tiled", False):
            raise ValueError("the backward takes a forward block with row-major operands (tiled=False)")
        if tiled and not fwd.fp8:
            raise ValueError("tiled backward operands are FP8 codes")
        self.tiled = bool(tiled)
        self._tn = B.FFN_TN_TILED if self.tiled else 0
        if grad_dtype not in ("e4m3", "e5m2"):
            raise ValueError(f"grad_dtype {grad_dtype!r}: need 'e4m3' or 'e5m2'")
        if grad_dtype == "e5m2" and not fwd.fp8:
            raise ValueError("an e5m2 gradient needs an FP8 block")
        self.grad_dtype = grad_dtype
        self.fuse_swiglu_bwd = fuse_swiglu_bwd
        self.concurrent = concurrent
        self._side = None   # the second stream, made on first use (default priority)
        self._wt_version = None   # weights_version the transposed weights were made from
        self.f = fwd
        N, C, H = fwd.N, fwd.C, fwd.H
        self.Np = _round_up(max(N, 1), 128)
        self.gu = _bf16(N, 2 * H)            # MlpUp
        self.dgu = self.gu if in_place else _bf16(N, 2 * H)   # dMlpUp
        self.dh = _bf16(N, H)                # dSwiGLU
        self.dy = _bf16(N, C)                # dLN2
        self.d_res = _bf16(N, C)             # dResAtt
        self.dw_d = _bf16(C, H)
        self.dw_gu = _bf16(2 * H, C)
        self.dw_norm = _f32(C)
        self.scratch = _f32(max(B.ffn_rmsnorm_bwd_scratch_bytes(N, C), 4) // 4)
        self.zero_once = zero_once
        # the gradient abs-max words, dMlpUp's and d_res's 16 bytes apart,
        # zeroed here (the zero-once form relies on that)
        self.am_tab = torch.zeros(8, dtype=torch.float32, device="cuda")
        self.am_dout, self.am_dgu, self.am_dres = _f32(1), self.am_tab[0:1], self.am_tab[4:5]
        if fwd.fp8 and self.tiled:
            t = B.ffn_tile_bytes
            self.qdout, self.s_dout = _u8(t(N, C)), _f32(1)
            self.qdgu, self.s_dgu = _u8(t(N, 2 * H)), _f32(1)
            self.wd_t, self.wgu_t = _u8(t(H, C)), _u8(t(C, 2 * H))
            self.dout_t, self.h_t = _u8(t(C, self.Np)), _u8(t(H, self.Np))
            self.dgu_t, self.y_t = _u8(t(2 * H, self.Np)), _u8(t(C, self.Np))
        elif fwd.fp8:
            self.qdout, self.s_dout = _u8(N, C), _f32(1)
            self.qdgu, self.s_dgu = _u8(N, 2 * H), _f32(1)
            self.wd_t, self.wgu_t = _u8(H, C), _u8(C, 2 * H)
            self.dout_t, self.h_t = _u8(C, self.Np), _u8(H, self.Np)
            self.dgu_t, self.y_t = _u8(2 * H, self.Np), _u8(C, self.Np)
        else:
            self.wd_t, self.wgu_t = _bf16(H, C), _bf16(C, 2 * H)
            self.dout_t, self.h_t = _bf16(C, self.Np), _bf16(H, self.Np)
            self.dgu_t, self.y_t = _bf16(2 * H, self.Np), _bf16(C, self.Np)
        self.zero_grads()

    def _swiglu_bwd_fused(self, a, a_scale, dtype, stream, flags=0):
        f = self.f
        if self.zero_once:
            am = self.am_dgu if f.fp8 else None
            fn = B.ffn_matmul_tn_swiglu_bwd_acc if am is not None else B.ffn_matmul_tn_swiglu_bwd
        else:
            am, fn = self.am_dgu, B.ffn_matmul_tn_swiglu_bwd
        fn(self.dgu, am, a, a_scale, self.wd_t, f.s_d if f.fp8 else None, self.gu, dtype, f.N, f.H, f.C, stream,
           flags=flags | self._tn)

    def _swiglu_bwd(self, stream):
        f = self.f
        if self.zero_once and f.fp8:
            B.ffn_swiglu_bwd_acc(self.dgu, self.am_dgu, self.dh, self.gu, f.N, f.H, stream)
        else:
            B.ffn_swiglu_bwd(self.dgu, None if self.zero_once else self.am_dgu, self.dh, self.gu, f.N, f.H, stream)

    def _transpose8(self, out, inp, rows, cols, ld_out, stream):
        """Transposed e4m3 codes (tiled when the products read tiled operands)."""
        if self.tiled:
            B.ffn_transpose_tiled(out, inp, rows, cols, ld_out, stream)
        else:
            B.ffn_transpose(out, inp, rows, cols, ld_out, 1, stream)

    def _quant_dout(self, d_out, E, stream):
        f = self.f
        if self.tiled:
            B.ffn_quant_transpose_tiled(self.dout_t, self.qdout, self.s_dout, d_out, self.am_dout, None, f.N, f.C,
                                        self.Np, stream, E)
        else:
            B.ffn_quant_transpose(self.dout_t, self.qdout, self.s_dout, d_out, self.am_dout, f.N, f.C, self.Np,
                                  stream, E)

    def _quant_dgu(self, E, stream):
        f = self.f
        if self.tiled:
            B.ffn_quant_transpose_tiled(self.dgu_t, self.qdgu, self.s_dgu, self.dgu, self.am_dgu,
                                        self.am_dres if self.zero_once else None, f.N, 2 * f.H, self.Np, stream, E)
        elif self.zero_once:
            B.ffn_quant_transpose_clear(self.dgu_t, self.qdgu, self.s_dgu, self.dgu, self.am_dgu, self.am_dres,
                                        f.N, 2 * f.H, self.Np, stream, E)
        else:
            B.ffn_quant_transpose(self.dgu_t, self.qdgu, self.s_dgu, self.dgu, self.am_dgu, f.N, 2 * f.H, self.Np,
                                  stream, E)

    def _rmsnorm_bwd(self, d_out, stream):
        f = self.f
        if self.zero_once and f.fp8:
            B.ffn_rmsnorm_bwd_acc(self.d_res, self.dw_norm, self.scratch, d_out, self.dy, self.r, f.w_norm, f.rstd,
                                  self.am_dres, self.am_dgu, f.N, f.C, stream)
        else:
            B.ffn_rmsnorm_bwd(self.d_res, self.dw_norm, self.scratch, d_out, self.dy, self.r, f.w_norm, f.rstd,
                              None if self.zero_once else self.am_dres, f.N, f.C, stream)

    def zero_grads(self):
        self.dw_d.zero_()
        self.dw_gu.zero_()
        self.dw_norm.zero_()

    def _weight_transposes(self, stream, mk):
        """W_down^T [H, C] and W_gu^T [C, 2H] (the codes for FP8), the b
        operands of the two data gradients, made only when the weights have
        changed since they were last made (backward_qmm transposes its
        weight on every call; within one weight update they do not change)."""
        f = self.f
        if self._wt_version == f.weights_version:
            return
        if f.fp8:
            self._transpose8(self.wd_t, f.w_d, f.C, f.H, f.C, stream)
            self._transpose8(self.wgu_t, f.w_gu, 2 * f.H, f.C, 2 * f.H, stream)
        else:
            B.ffn_transpose(self.wd_t, f.w_d, f.C, f.H, f.C, 2, stream)
            B.ffn_transpose(self.wgu_t, f.w_gu, 2 * f.H, f.C, 2 * f.H, 2, stream)
        self._wt_version = f.weights_version
        mk("transpose_weights")

    def forward(self, inp, addend, stream=None):
        """The block forward with the up-projection output kept: RMSNorm,
        (quantise y), gate+up GEMM to gu [N, 2H], SwiGLU with its abs-max,
        (quantise h), down GEMM.  Returns the down output [N, C]."""
        f = self.f
        N, C, H = f.N, f.C, f.H
        B.ffn_rmsnorm_fwd(f.y, f.rstd, f.r if addend is not None else None, f.am_y, inp, addend, f.w_norm, f.eps,
                          N, C, stream)
        self.r = f.r if addend is not None else inp
        if f.fp8:
            B.ffn_quant_absmax(f.qy, f.s_y, f.am_y, f.y, N * C, 0, stream)
            B.ffn_gateup(self.gu, None, f.qy, f.s_y, f.w_gu, f.s_gu, B.FFN_E4M3, 0, N, C, H, stream)
            B.ffn_swiglu(f.h, f.am_h, self.gu, N, H, stream)
            B.ffn_quant_absmax(f.qh, f.s_h, f.am_h, f.h, N * H, 0, stream)
            B.ffn_down(f.out, f.qh, f.s_h, f.w_d, f.s_d, B.FFN_E4M3, N, H, C, stream)
        else:
            B.ffn_gateup(self.gu, None, f.y, None, f.w_gu, None, B.FFN_BF16, 0, N, C, H, stream)
            B.ffn_swiglu(f.h, f.am_h, self.gu, N, H, stream)
            B.ffn_down(f.out, f.h, None, f.w_d, None, B.FFN_BF16, N, H, C, stream)
        return f.out

    def backward(self, d_out, stream=None, mark=None, d_out_absmax=None):
        """Backward from d_out [N, C] (the gradient of the block's output
        residual stream, DResFFN) after ``forward``.  Returns d_res (DResAtt);
        dw_d, dw_gu (bf16) and dw_norm (fp32) accumulate.  d_out_absmax: the
        abs-max of d_out when its producer already wrote it (the upstream
        ``ffn_rmsnorm_bwd`` does, as the trainer's rmsnorm_backward does for
        DResFFN); None computes it here.  mark(label), when given, is called
        after each phase (for per-phase timing)."""
        if self.concurrent and mark is None:
            return self._backward_concurrent(d_out, stream, d_out_absmax)
        f = self.f
        N, C, H, Np = f.N, f.C, f.H, self.Np
        dgu = self.dgu
        mk = mark or (lambda label: None)
        self._weight_transposes(stream, mk)
        if f.fp8:
            # gradient codes (the TN matmuls' a operand) in the grad dtype
            E = B.FFN_E5M2 if self.grad_dtype == "e5m2" else B.FFN_E4M3
            # backward_qmm through the down projection (input h, weight [C, H])
            # the gradient's codes in both layouts from one read
            if d_out_absmax is None:
                B.ffn_quant_absmax(self.qdout, self.s_dout, self.am_dout, d_out, N * C, 1, stream)
            else:
                self.am_dout = d_out_absmax
            self._quant_dout(d_out, E, stream)
            mk("quant_dout")
            TL = self._tn
            if self.fuse_swiglu_bwd:
                self._swiglu_bwd_fused(self.qdout, self.s_dout, E, stream)
                mk("dx_down_swiglu_bwd")
            else:
                B.ffn_matmul_tn(self.dh, self.qdout, self.s_dout, self.wd_t, f.s_d, E, TL, N, H, C, stream)
                mk("dx_down")
            self._transpose8(self.h_t, f.qh, N, H, Np, stream)
            mk("transpose_down_operands")
            B.ffn_matmul_tn(self.dw_d, self.dout_t, self.s_dout, self.h_t, f.s_h, E, 1 | TL, C, H, Np, stream)
            mk("dw_down")
            if not self.fuse_swiglu_bwd:
                self._swiglu_bwd(stream)
                mk("swiglu_bwd")
            # backward_qmm through the up projection (input y, weight [2H, C])
            self._quant_dgu(E, stream)
            mk("quant_dgu")
            B.ffn_matmul_tn(self.dy, self.qdgu, self.s_dgu, self.wgu_t, f.s_gu, E, TL, N, C, 2 * H, stream)
            mk("dx_up")
            self._transpose8(self.y_t, f.qy, N, C, Np, stream)
            mk("transpose_up_operands")
            B.ffn_matmul_tn(self.dw_gu, self.dgu_t, self.s_dgu, self.y_t, f.s_y, E, 1 | TL, 2 * H, C, Np, stream)
            mk("dw_up")
        else:
            Bf = B.FFN_BF16
            if self.fuse_swiglu_bwd:
                self._swiglu_bwd_fused(d_out, None, Bf, stream)
                mk("dx_down_swiglu_bwd")
            else:
                B.ffn_matmul_tn(self.dh, d_out, None, self.wd_t, None, Bf, 0, N, H, C, stream)
                mk("dx_down")
            B.ffn_transpose(self.dout_t, d_out, N, C, Np, 2, stream)
            B.ffn_transpose(self.h_t, f.h, N, H, Np, 2, stream)
            mk("transpose_down_operands")
            B.ffn_matmul_tn(self.dw_d, self.dout_t, None, self.h_t, None, Bf, 1, C, H, Np, stream)
            mk("dw_down")
            if not self.fuse_swiglu_bwd:
                self._swiglu_bwd(stream)
                mk("swiglu_bwd")
            B.ffn_matmul_tn(self.dy, dgu, None, self.wgu_t, None, Bf, 0, N, C, 2 * H, stream)
            mk("dx_up")
            B.ffn_transpose(self.dgu_t, dgu, N, 2 * H, Np, 2, stream)
            B.ffn_transpose(self.y_t, f.y, N, C, Np, 2, stream)
            mk("transpose_up_operands")
            B.ffn_matmul_tn(self.dw_gu, self.dgu_t, None, self.y_t, None, Bf, 1, 2 * H, C, Np, stream)
            mk("dw_up")
        # rmsnorm_backward: DResAtt = DResFFN + the RMSNorm input's gradient
        self._rmsnorm_bwd(d_out, stream)
        mk("rmsnorm_bwd")
        return self.d_res

    def _backward_concurrent(self, d_out, stream, d_out_absmax):
        """backward() with the weight gradients on a second stream: after the
        down projection's operands are ready the second stream transposes h
        and runs dW_d, while this stream runs the data gradient (with the
        SwiGLU backward), quantises dMlpUp and transposes the up weight; then
        the second stream transposes y and runs dW_gu while this one runs the
        up projection's data gradient and the RMSNorm backward."""
        f = self.f
        N, C, H, Np = f.N, f.C, f.H, self.Np
        dgu = self.dgu
        main = stream if stream is not None else torch.cuda.current_stream()
        if self._side is None:
            self._side = torch.cuda.Stream()
            self._ev = [torch.cuda.Event() for _ in range(3)]
        side = self._side
        T, ACC = B.FFN_TN_TILE_GRID, B.FFN_TN_ACCUMULATE

        def fork(k):
            self._ev[k].record(main)
            side.wait_event(self._ev[k])

        self._weight_transposes(main, lambda label: None)

        if f.fp8:
            E = B.FFN_E5M2 if self.grad_dtype == "e5m2" else B.FFN_E4M3
            if d_out_absmax is None:
                B.ffn_quant_absmax(self.qdout, self.s_dout, self.am_dout, d_out, N * C, 1, main)
            else:
                self.am_dout = d_out_absmax
            self._quant_dout(d_out, E, main)
            TL = self._tn
            fork(0)
            self._transpose8(self.h_t, f.qh, N, H, Np, side)
            B.ffn_matmul_tn(self.dw_d, self.dout_t, self.s_dout, self.h_t, f.s_h, E, ACC | T | TL, C, H, Np, side)
            if self.fuse_swiglu_bwd:
                self._swiglu_bwd_fused(self.qdout, self.s_dout, E, main, flags=T)
            else:
                B.ffn_matmul_tn(self.dh, self.qdout, self.s_dout, self.wd_t, f.s_d, E, T | TL, N, H, C, main)
                self._swiglu_bwd(main)
            self._quant_dgu(E, main)
            fork(1)
            self._transpose8(self.y_t, f.qy, N, C, Np, side)
            B.ffn_matmul_tn(self.dw_gu, self.dgu_t, self.s_dgu, self.y_t, f.s_y, E, ACC | T | TL, 2 * H, C, Np, side)
            B.ffn_matmul_tn(self.dy, self.qdgu, self.s_dgu, self.wgu_t, f.s_gu, E, T | TL, N, C, 2 * H, main)
        else:
            Bf = B.FFN_BF16
            fork(0)
            B.ffn_transpose(self.dout_t, d_out, N, C, Np, 2, side)
            B.ffn_transpose(self.h_t, f.h, N, H, Np, 2, side)
            B.ffn_matmul_tn(self.dw_d, self.dout_t, None, self.h_t, None, Bf, ACC | T, C, H, Np, side)
            if self.fuse_swiglu_bwd:
                self._swiglu_bwd_fused(d_out, None, Bf, main, flags=T)
            else:
                B.ffn_matmul_tn(self.dh, d_out, None, self.wd_t, None, Bf, T, N, H, C, main)
                self._swiglu_bwd(main)
            fork(1)
            B.ffn_transpose(self.dgu_t, dgu, N, 2 * H, Np, 2, side)
            B.ffn_transpose(self.y_t, f.y, N, C, Np, 2, side)
            B.ffn_matmul_tn(self.dw_gu, self.dgu_t, None, self.y_t, None, Bf, ACC | T, 2 * H, C, Np, side)
            B.ffn_matmul_tn(self.dy, dgu, None, self.wgu_t, None, Bf, T, N, C, 2 * H, main)
        self._rmsnorm_bwd(d_out, main)
        # the second stream's work joins this stream's
        self._ev[2].record(side)
        main.wait_event(self._ev[2])
        return self.d_res
