"""The FFN block, step by step, as plain numpy.  TEST INFRASTRUCTURE ONLY.

What is computed follows three pages:

* llmq ``llama_model.cpp`` — ``LLamaModel::_forward_block`` (the FFN half:
  ``fused_residual_rmsnorm_forward`` into LN2, ``forward_qmm`` with the
  ``[2H, C]`` up weight, ``swiglu_forward``, ``forward_qmm`` with the
  ``[C, H]`` down weight), ``LLamaModel::forward`` (the next layer's fused
  residual RMSNorm closes the block; ``fill_zero`` of the abs-max table) and
  ``forward_qmm`` (quantise the input with its abs-max, then a matmul scaled
  by the weight's and the input's scales);
* llmq ``llama_run_state.cpp`` — ``allocate_basic_fwd_tensors`` (rstd is an
  fp32 ``[B, T]`` tensor, ``mlp_up`` is ``[B, T, 2H]``, the SwiGLU output is
  ``[B, T, H]``; the RMSNorm output may overwrite its own input) and
  ``allocate_fwd_quant_tensors`` (e4m3 copies, two fp32 abs-max/scale slots
  per quantised tensor);
* metrale ``dense_ffn_decode.rs`` — ``DenseFfnLayer::forward``, FP8 arm
  (``w8a16_gemv_dual`` with per-row scales, ``silu_mul`` in place, then
  ``w8a16_gemv`` for the down projection: the split-SiLU arm, the default).

Where the pages leave a step open the reading taken is stated in the
docstring.  Shapes: N rows, C hidden, H intermediate; all matrices row-major;
weights are ``[out, in]``.

Precision: sums and dot products in fp64 (numpy), one rounding to each stored
type; the elementwise products the block takes in fp32 (the RMSNorm output's
two products, the product that decides a code) are fp32 products here too.
bf16 tensors enter and leave as uint16 bit patterns, e4m3 as uint8, fp32
scalars and vectors as float32.
"""

import numpy as np

from .codecs import bf16_bits_to_f64, f64_to_bf16_bits, bf16_round, e4m3_decode, e4m3_encode, E4M3_MAX, FP8_FORMATS


def _f32(x):
    return np.float32(x)


def residual_add(a_bits, b_bits):
    """r = bf16(a + b): the residual stream update that the fused RMSNorm
    writes to its residual output (llama_model.cpp, ``LLamaModel::forward`` and
    ``_forward_block``, first argument of ``fused_residual_rmsnorm_forward``).
    Reading: exact sum, one rounding to bf16."""
    return f64_to_bf16_bits(bf16_bits_to_f64(a_bits) + bf16_bits_to_f64(b_bits))


def rms_rstd(r_bits, eps):
    """rstd_i = fp32( 1 / sqrt( sum_j r_ij^2 / C + eps ) ) for a bf16 [N, C]
    tensor (the rstd that ``fused_residual_rmsnorm_forward`` saves, fp32
    ``[B, T]``).  Reading: eps inside the square root, mean by division by C."""
    r = bf16_bits_to_f64(r_bits)
    C = r.shape[-1]
    ms = np.sum(r * r, axis=-1) / C
    return (1.0 / np.sqrt(ms + np.float64(_f32(eps)))).astype(np.float32)


def rms_apply(r_bits, rstd, weight_bits):
    """y_ij = bf16( fp32( fp32(r_ij * rstd_i) * w_j ) ) with the stored fp32
    rstd, and max |y| over the stored bf16 y.  The two products are fp32
    products (the block's arithmetic is fp32), then one rounding to bf16.
    Returns (y_bits, absmax float32)."""
    r = bf16_bits_to_f64(r_bits).astype(np.float32)
    w = bf16_bits_to_f64(weight_bits).astype(np.float32)
    t = r * np.asarray(rstd, np.float32)[..., None]
    y32 = t * w[None, :]
    y = bf16_round(y32.astype(np.float64))
    absmax = _f32(np.max(np.abs(y))) if y.size else _f32(0.0)
    return f64_to_bf16_bits(y), absmax


def rmsnorm_fwd(inp_bits, addend_bits, weight_bits, eps):
    """Fused residual add + RMSNorm with saved rstd and the output's abs-max.

    llama_model.cpp, ``LLamaModel::_forward_block``: ``fused_residual_rmsnorm_forward(
    ResidualAtt, LN2, LN2_Rstd, residual, AttO, LN2_w, LN2 abs-max, eps, B*T, C)``;
    without an addend it is ``rmsnorm_forward`` (``LLamaModel::forward``, layer 0).

      r_i    = bf16(inp_i + addend_i)            (r = inp when there is no addend)
      rstd_i = fp32( 1 / sqrt( sum_j r_ij^2 / C + eps ) )
      y_ij   = bf16( (r_ij * rstd_i) * w_j )     (fp32 products, rstd as stored)
      absmax = max_ij |y_ij|                     over the stored bf16 y

    Readings: eps inside the square root, mean by division by C; y from the
    rounded r and the stored fp32 rstd; the abs-max is taken over the rounded
    output, the tensor the quantiser reads.

    Returns (residual_bits or None, y_bits, rstd float32[N], absmax float32).
    """
    if addend_bits is None:
        r_bits = None
        r = np.asarray(inp_bits)
    else:
        r_bits = residual_add(inp_bits, addend_bits)
        r = r_bits
    rstd = rms_rstd(r, eps)
    y, absmax = rms_apply(r, rstd, weight_bits)
    return r_bits, y, rstd, absmax


def absmax_of(bits):
    """max |x| over a bf16 tensor, as fp32 (exact: a bf16 value is an fp32 value).
    llama_model.cpp, ``_forward_block``: ``abs_max(...)``.  A NaN element makes
    the abs-max NaN."""
    x = bf16_bits_to_f64(bits)
    return _f32(np.max(np.abs(x))) if x.size else _f32(0.0)


def scales_from_absmax(absmax, fmt="e4m3"):
    """(scale, inv) for a per-tensor abs-max.

    Reading (the pages only name a ``scale()`` slot next to ``abs_max()``,
    llama_run_state.cpp ``allocate_fwd_quant_tensors``): scale is the
    dequantisation factor absmax/max and inv = max/absmax multiplies the input,
    with max the format's largest finite value (448 for e4m3, 57344 for e5m2);
    both are IEEE fp32 quotients.  An all-zero tensor (absmax == 0) gets
    scale = inv = 1; a NaN abs-max (a NaN anywhere in the tensor) gives NaN for
    both, so every code of the tensor is a NaN code.
    """
    fmax = FP8_FORMATS[fmt][2]
    am = np.float64(_f32(absmax))
    if am != 0:
        return _f32(am / fmax), _f32(fmax / am)
    return _f32(1.0), _f32(1.0)


def quant_absmax(x_bits, absmax=None, fmt="e4m3"):
    """Per-tensor abs-max e4m3 quantisation (llama_model.cpp, ``forward_qmm``:
    ``quantize_with_abs_max(inp.Quant, inp.Quant.scale(), inp.Value,
    inp.Quant.abs_max(), ...)``).  With absmax None it is computed first.

      q = e4m3( fp32( x * inv ) ),   scale = absmax / 448

    The product that decides the code is taken in fp32.  fmt "e5m2" gives the
    other FP8 gradient format, with its own largest value.
    Returns (codes uint8, scale float32, absmax float32).
    """
    if absmax is None:
        absmax = absmax_of(x_bits)
    scale, inv = scales_from_absmax(absmax, fmt)
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)
    q = FP8_FORMATS[fmt][0](x32 * inv)
    return q, scale, _f32(absmax)


def quant_rows(w_bits):
    """Per-row abs-max e4m3 quantisation of a weight matrix ``[rows, cols]``:
    the ``QuantizedWeight { weight, row_scale }`` layout of the FP8 decode
    weights (dense_ffn_decode.rs, ``DenseFfnLayer::forward``, FP8 arm).  Each
    row is quantised exactly as ``quant_absmax`` quantises a tensor.
    Returns (codes uint8 [rows, cols], row_scale float32 [rows])."""
    w_bits = np.asarray(w_bits)
    q = np.empty(w_bits.shape, dtype=np.uint8)
    s = np.empty(w_bits.shape[0], dtype=np.float32)
    for i in range(w_bits.shape[0]):
        q[i], s[i], _ = quant_absmax(w_bits[i])
    return q, s


def _matmul_nt(x, w):
    """sum_k x[n,k] * w[o,k] in fp64 (a library matmul on float64 operands)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def gemm_bf16(x_bits, w_bits):
    """out[n,o] = bf16( sum_k x[n,k] * W[o,k] ) — ``matmul(out, weight, inp, ...,
    OC, B*T, C, EMMTranspose::TN)`` in ``forward_qmm`` (llama_model.cpp) when
    weight and input share the bf16 dtype.  Column-major TN with the weight as
    A is the row-major product X * W^T."""
    return f64_to_bf16_bits(_matmul_nt(bf16_bits_to_f64(x_bits), bf16_bits_to_f64(w_bits)))


def gemm_fp8(qx, sx, qw, sw):
    """out[n,o] = bf16( (sum_k dec(qx[n,k]) * dec(qw[o,k])) * fp32(sx * sw) ) —
    the scaled matmul of ``forward_qmm`` (llama_model.cpp) with
    ``weight.scale()`` and ``inp.Quant.scale()``.  Reading: the two scales are
    multiplied once in fp32 and applied to the finished sum."""
    s = np.float64(_f32(np.float64(_f32(sx)) * np.float64(_f32(sw))))
    return f64_to_bf16_bits(_matmul_nt(e4m3_decode(qx), e4m3_decode(qw)) * s)


def silu(g):
    """silu(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gu_bits):
    """h[n,j] = bf16( silu(g) * u ) with g = GU[n, j], u = GU[n, H + j], and
    absmax(h) — ``swiglu_forward(SwiGLu, MlpUp, SwiGLu abs-max, B, T, D)``
    (llama_model.cpp, ``_forward_block``).  Reading: the first H columns of the
    ``[N, 2H]`` up-projection output are the gate, the last H the up half.
    Returns (h_bits, absmax float32)."""
    gu = bf16_bits_to_f64(gu_bits)
    H = gu.shape[-1] // 2
    h = bf16_round(silu(gu[..., :H]) * gu[..., H:])
    am = _f32(np.max(np.abs(h))) if h.size else _f32(0.0)
    return f64_to_bf16_bits(h), am


def decode_dual(x_bits, wg, sg, wu, su):
    """The dual gate/up GEMV with the SiLU product (dense_ffn_decode.rs,
    ``DenseFfnLayer::forward``, FP8 arm: ``w8a16_gemv_dual`` then ``silu_mul``):

      g[m,n] = bf16( sg[n] * sum_k dec(Wg[n,k]) * x[m,k] ),  u likewise
      h[m,n] = bf16( silu(g) * u )

    Readings: the intermediates are bf16 (16-bit activations); each row scale
    multiplies the finished dot product.  Returns h_bits [M, H]."""
    x = bf16_bits_to_f64(x_bits)
    g = bf16_round(_matmul_nt(x, e4m3_decode(wg)) * np.asarray(sg, np.float32).astype(np.float64)[None, :])
    u = bf16_round(_matmul_nt(x, e4m3_decode(wu)) * np.asarray(su, np.float32).astype(np.float64)[None, :])
    return f64_to_bf16_bits(silu(g) * u)


def decode_down(h_bits, wd, sd):
    """The down GEMV (``w8a16_gemv`` with the down weight, n_out = hidden,
    k_in = intermediate): y[m,c] = bf16( sd[c] * sum_n dec(Wd[c,n]) * h[m,n] )."""
    h = bf16_bits_to_f64(h_bits)
    return f64_to_bf16_bits(_matmul_nt(h, e4m3_decode(wd)) * np.asarray(sd, np.float32).astype(np.float64)[None, :])


def decode_gemv(x_bits, wg, sg, wu, su, wd, sd):
    """Single-token (or few-token) FP8 W8A16 decode FFN, split-SiLU arm (the
    default arm of dense_ffn_decode.rs, ``DenseFfnLayer::forward``, FP8 arm):
    ``decode_dual`` then ``decode_down``.  Returns (y_bits [M, C], h_bits [M, H])."""
    h = decode_dual(x_bits, wg, sg, wu, su)
    return decode_down(h, wd, sd), h


def decode_gemv_bf16(x_bits, wg_bits, wu_bits, wd_bits):
    """Few-token decode FFN with bf16 weights (dense_ffn_decode.rs,
    ``DenseFfnLayer::forward``, bf16 arm: ``dense_gemv`` for gate and for up,
    ``silu_mul``, ``dense_gemv`` for down):

      g = bf16( sum_k Wg[n,k] x[m,k] ),  u likewise,  h = bf16( silu(g) * u )
      y = bf16( sum_n Wd[c,n] h[m,n] )

    Returns (y_bits [M, C], h_bits [M, H])."""
    g = bf16_bits_to_f64(gemm_bf16(x_bits, wg_bits))
    u = bf16_bits_to_f64(gemm_bf16(x_bits, wu_bits))
    h = f64_to_bf16_bits(silu(g) * u)
    return gemm_bf16(h, wd_bits), h


def block_forward(inp, addend, w_norm, w_gu, w_d, eps, fp8=False):
    """One FFN block as ``_forward_block`` runs it from LN2 on, plus the closing
    residual that the next fused RMSNorm applies (``LLamaModel::forward``).

    inp, addend: bf16 [N, C] (residual stream and attention output);
    w_norm: bf16 [C]; w_gu: bf16 [2H, C] (gate rows, then up rows);
    w_d: bf16 [C, H].  With fp8=True the weights are quantised per tensor with
    their own abs-max (the weight scales come from the weights' abs-max, as the
    optimizer step's abs-max output feeds them) and both activations are
    quantised per tensor before their matmul (``forward_qmm``).

    Returns a dict with every intermediate.
    """
    out = {}
    r, y, rstd, am_y = rmsnorm_fwd(inp, addend, w_norm, eps)
    r_vals = inp if r is None else r
    out.update(residual=r, rms_input=r_vals, y=y, rstd=rstd, absmax_y=am_y)
    if not fp8:
        gu = gemm_bf16(y, w_gu)
        h, am_h = swiglu(gu)
        d = gemm_bf16(h, w_d)
    else:
        qw_gu, s_gu, _ = quant_absmax(w_gu)
        qw_d, s_d, _ = quant_absmax(w_d)
        qy, s_y, _ = quant_absmax(y, am_y)
        gu = gemm_fp8(qy, s_y, qw_gu, s_gu)
        h, am_h = swiglu(gu)
        qh, s_h, _ = quant_absmax(h, am_h)
        d = gemm_fp8(qh, s_h, qw_d, s_d)
        out.update(qw_gu=qw_gu, s_gu=s_gu, qw_d=qw_d, s_d=s_d, qy=qy, s_y=s_y, qh=qh, s_h=s_h)
    out.update(gu=gu, h=h, absmax_h=am_h, down=d)
    out["next_residual"] = residual_add(r_vals, d)
    return out
