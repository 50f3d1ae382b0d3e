"""The FFN block's backward pass, step by step, as plain numpy.  TEST
INFRASTRUCTURE ONLY (see the package docstring).

What is computed follows llmq ``llama_model.cpp``:

* ``LLamaModel::_backward_block`` (its FFN half): ``backward_qmm`` through the
  down projection (the gradient of the block output gives the SwiGLU output's
  gradient and the down weight's gradient), ``swiglu_backward`` (the gradient
  of the ``[B, T, 2H]`` up-projection output, with its abs-max), ``backward_qmm``
  through the ``[2H, C]`` up weight, then ``rmsnorm_backward``, which adds the
  RMSNorm input's gradient to the residual stream's gradient and accumulates
  the norm weight's gradient;
* ``backward_qmm``: with bf16 weights ``dinp = dout * W`` (NN) and
  ``dweight (+)= dout^T * inp`` (NT); with e4m3 weights the output gradient is
  quantised per tensor with its abs-max, the weight, the (forward-quantised)
  input and the quantised gradient are transposed, and both products run as
  scaled TN matmuls whose scales are the two operands' scales.

The pages call ``swiglu_backward`` and ``rmsnorm_backward`` without showing
their bodies; they are the derivatives of the forward steps, written out here
(the readings are stated in each docstring).  Precision as in ``ffn.py``: sums
in fp64, one rounding to each stored type.
"""

import numpy as np

from .codecs import bf16_bits_to_f64, f64_to_bf16_bits, bf16_round, FP8_FORMATS
from .ffn import _f32, _matmul_nt, absmax_of, quant_absmax


def sigmoid(g):
    """1 / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def swiglu_bwd(dh_bits, gu_bits):
    """Gradient of h = silu(g) * u (llama_model.cpp, ``_backward_block``:
    ``swiglu_backward(DMlpUp, DSwiGLU, MlpUp, DMlpUp abs-max, B, T, D)``).

      dg[n,j] = bf16( dh * u * s * (1 + g * (1 - s)) ),  s = sigmoid(g)
      du[n,j] = bf16( dh * g * s )

    written to ``[N, 2H]`` in the forward's layout (gate columns, then up
    columns), and max |dgu| over the stored bf16 values.  Reading: the exact
    derivative of the forward's fp32 formula, one rounding per output.
    Returns (dgu_bits [N, 2H], absmax float32)."""
    dh = bf16_bits_to_f64(dh_bits)
    gu = bf16_bits_to_f64(gu_bits)
    H = gu.shape[-1] // 2
    g, u = gu[..., :H], gu[..., H:]
    s = sigmoid(g)
    dg = bf16_round(dh * u * s * (1.0 + g * (1.0 - s)))
    du = bf16_round(dh * g * s)
    dgu = np.concatenate([dg, du], axis=-1)
    am = _f32(np.max(np.abs(dgu))) if dgu.size else _f32(0.0)
    return f64_to_bf16_bits(dgu), am


def rmsnorm_bwd(dresidual_bits, dy_bits, r_bits, w_bits, rstd, dweight=None):
    """Backward of ``y = bf16(r * rstd * w)`` (llama_model.cpp,
    ``_backward_block``: ``rmsnorm_backward(DResAtt, LN2_w grad, scratch,
    DResFFN, DLN2, ResidualAtt, LN2_w, LN2_Rstd, DResAtt abs-max, B, T, C)``;
    the comment beside it: the result is added to the residual stream's
    gradient).

      xh = r * rstd,  gy = dy * w,  m = sum_j gy_j * xh_j / C
      dinp[n,j] = bf16( dresidual[n,j] + rstd * (gy_j - xh_j * m) )
      dweight[j] = fp32( dweight[j] + sum_n dy[n,j] * xh[n,j] )
      absmax = max |dinp|

    Readings: the saved fp32 rstd is used as the forward used it (the
    derivative of rstd with respect to r is taken through the formula
    rstd = (sum r^2 / C + eps)^-1/2, which gives the -xh * m term); dinp may
    overwrite dresidual; the weight gradient accumulates in fp32 (the trainer
    zeroes gradients before the first micro-step and accumulates afterwards).
    dweight None means a zero accumulator.
    Returns (dinp_bits, dweight float32 [C], absmax float32)."""
    r = bf16_bits_to_f64(r_bits)
    dy = bf16_bits_to_f64(dy_bits)
    w = bf16_bits_to_f64(w_bits)
    dres = bf16_bits_to_f64(dresidual_bits)
    rs = np.asarray(rstd, np.float32).astype(np.float64)[..., None]
    C = r.shape[-1]
    xh = r * rs
    gy = dy * w[None, :]
    m = np.sum(gy * xh, axis=-1, keepdims=True) / C
    dinp = bf16_round(dres + rs * (gy - xh * m))
    old = np.zeros(C) if dweight is None else np.asarray(dweight, np.float32).astype(np.float64)
    dw = (old + np.sum(dy * xh, axis=0)).astype(np.float32)
    am = _f32(np.max(np.abs(dinp))) if dinp.size else _f32(0.0)
    return f64_to_bf16_bits(dinp), dw, am


def transpose(x):
    """out[c, r] = x[r, c] (``transpose`` in ``backward_qmm``): a copy, no
    arithmetic."""
    return np.ascontiguousarray(np.asarray(x).T)


def matmul_tn(a, b, a_scale=None, b_scale=None, accumulate=None, a_fmt="e4m3", b_fmt="e4m3"):
    """out[m, n] = bf16( acc[m,n] + (sum_k A[m,k] * B[n,k]) * s ) — the TN
    matmul of ``backward_qmm`` in row-major terms (both operands K-contiguous).
    bf16 operands when the scales are None (s = 1), else FP8 codes (a_fmt,
    b_fmt: "e4m3" or "e5m2") with s = fp32(a_scale * b_scale).  ``accumulate``
    is the bf16 output it adds to (the ``accumulate_gradient`` flag); None
    means a plain store.  Reading: the accumulation happens before the single
    rounding to bf16, as a matmul's ``C + A*B`` does in its fp32 compute type."""
    if a_scale is None:
        prod = _matmul_nt(bf16_bits_to_f64(a), bf16_bits_to_f64(b))
    else:
        s = np.float64(_f32(np.float64(_f32(a_scale)) * np.float64(_f32(b_scale))))
        prod = _matmul_nt(FP8_FORMATS[a_fmt][1](a), FP8_FORMATS[b_fmt][1](b)) * s
    if accumulate is not None:
        prod = prod + bf16_bits_to_f64(accumulate)
    return f64_to_bf16_bits(prod)


def linear_bwd(dy, x, w, fp8=False, dy_absmax=None, qx=None, sx=None, qw=None, sw=None, dw_acc=None,
               grad_fmt="e4m3"):
    """``backward_qmm`` for out = x * W^T with x ``[N, C]``, W ``[OC, C]``,
    dy ``[N, OC]``.  Returns a dict with dx ``[N, C]`` and dw ``[OC, C]``
    (bf16 bits) and, for FP8, the quantised gradient.

    bf16:  dx = bf16( dy * W ),  dw = bf16( dw_acc + dy^T * x )
    FP8:   qdy, sdy = quantise(dy, dy_absmax) (the abs-max its producer wrote);
           dx = bf16( (qdy * qW) * (sW * sdy) )          (W transposed, TN)
           dw = bf16( dw_acc + (qdy^T * qx) * (sx * sdy) )  (both transposed, TN)
    qx/sx: the input's forward codes and scale (reused, as ``reuse_inp`` does);
    qw/sw: the weight's codes and scale (e4m3).  grad_fmt: the gradient's
    codes, e4m3 or e5m2 (the two FP8 grad dtypes the pages allow), each with
    its own largest value in the scale."""
    if not fp8:
        wt = transpose(w)
        dx = matmul_tn(dy, wt)
        dw = matmul_tn(transpose(dy), transpose(x), accumulate=dw_acc)
        return {"dx": dx, "dw": dw}
    if dy_absmax is None:
        dy_absmax = absmax_of(dy)
    qdy, sdy, _ = quant_absmax(dy, dy_absmax, grad_fmt)
    dx = matmul_tn(qdy, transpose(qw), sdy, sw, a_fmt=grad_fmt)
    dw = matmul_tn(transpose(qdy), transpose(qx), sdy, sx, accumulate=dw_acc, a_fmt=grad_fmt)
    return {"dx": dx, "dw": dw, "qdy": qdy, "sdy": sdy}


def block_backward(fwd, d_out, w_norm, w_gu, w_d, fp8=False, acc=None, grad_fmt="e4m3"):
    """The FFN half of ``LLamaModel::_backward_block``.

    fwd: ``block_forward``'s dict for the same inputs (the RMSNorm input, y,
    rstd, gu, h and, for FP8, the weight and activation codes); d_out: bf16
    ``[N, C]``, the gradient of the block's output residual stream (DResFFN),
    which reaches the down projection and passes the residual connection.
    acc: optional dict of gradient accumulators (``dw_d``, ``dw_gu`` bf16,
    ``dw_norm`` fp32).  Returns a dict with every intermediate and
    ``d_residual`` (DResAtt, the gradient handed to the attention half).

      dh            = down backward of d_out        (dSwiGLU [N, H]); dW_d
      dgu, am_dgu   = swiglu_bwd(dh, gu)            (dMlpUp [N, 2H])
      dy            = up backward of dgu            (dLN2 [N, C]); dW_gu
      d_residual    = rmsnorm_bwd(d_out, dy, r, ...); dw_norm

    FP8: d_out is quantised with its own abs-max, dgu with swiglu_bwd's, both
    to grad_fmt codes (e4m3 or e5m2).
    """
    acc = acc or {}
    out = {}
    r = fwd["rms_input"]
    down = linear_bwd(d_out, fwd["h"], w_d, fp8, qx=fwd.get("qh"), sx=fwd.get("s_h"), qw=fwd.get("qw_d"),
                      sw=fwd.get("s_d"), dw_acc=acc.get("dw_d"), grad_fmt=grad_fmt)
    dh = down["dx"]
    dgu, am_dgu = swiglu_bwd(dh, fwd["gu"])
    up = linear_bwd(dgu, fwd["y"], w_gu, fp8, dy_absmax=am_dgu, qx=fwd.get("qy"), sx=fwd.get("s_y"),
                    qw=fwd.get("qw_gu"), sw=fwd.get("s_gu"), dw_acc=acc.get("dw_gu"), grad_fmt=grad_fmt)
    dres, dw_norm, am_res = rmsnorm_bwd(d_out, up["dx"], r, w_norm, fwd["rstd"], acc.get("dw_norm"))
    out.update(dh=dh, dw_d=down["dw"], dgu=dgu, absmax_dgu=am_dgu, dy=up["dx"], dw_gu=up["dw"],
               d_residual=dres, dw_norm=dw_norm, absmax_d_residual=am_res)
    if fp8:
        out.update(qd_out=down["qdy"], sd_out=down["sdy"], qdgu=up["qdy"], sdgu=up["sdy"])
    return out
