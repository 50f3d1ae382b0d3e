"""CPU oracle for the dense SwiGLU FFN block and its FP8 decode form.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``transformer_ffn_block_residual_amd/csrc`` and imports nothing
from that package.

Two independent implementations of the same definitions:

* this package's numpy modules (``codecs``, ``ffn``, ``backward``): reductions
  and dot products in fp64, every value the pages store (bf16 activations,
  fp32 rstd and scales, e4m3 codes) rounded exactly once to its storage type;
  the elementwise products the block takes in fp32 (the RMSNorm output, the
  product that decides an FP8 code) are fp32 products;
* ``cpp`` (``ffn_oracle.cpp``, plain C++ built with the host compiler): the
  forward block and the FP8 decode in fp32 with a fixed 16-way summation
  order and ``std::thread`` over output rows, fast enough for whole full-size
  outputs and the CPU baseline.

Bit patterns cross both interfaces as integer arrays (bf16 as uint16, e4m3 as
uint8, fp32 as float32) so that nothing depends on another library's rounding.

Parity status of each function is recorded in its docstring; every function
here is pinned by a ``-m "not gpu"`` test under ``tests/`` against closed
forms, brute force or an independent library routine.
"""

from .codecs import (
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    bf16_round,
    e4m3_decode,
    e4m3_encode,
    E4M3_MAX,
    e5m2_decode,
    e5m2_encode,
    E5M2_MAX,
)
from .ffn import (
    residual_add,
    rms_rstd,
    rms_apply,
    rmsnorm_fwd,
    absmax_of,
    scales_from_absmax,
    quant_absmax,
    quant_rows,
    gemm_bf16,
    gemm_fp8,
    silu,
    swiglu,
    decode_dual,
    decode_down,
    decode_gemv,
    decode_gemv_bf16,
    block_forward,
)
from .backward import (
    sigmoid,
    swiglu_bwd,
    rmsnorm_bwd,
    transpose,
    matmul_tn,
    linear_bwd,
    block_backward,
)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "bf16_round", "e4m3_decode",
    "e4m3_encode", "E4M3_MAX", "e5m2_decode", "e5m2_encode", "E5M2_MAX", "residual_add", "rms_rstd", "rms_apply", "rmsnorm_fwd",
    "absmax_of", "scales_from_absmax", "quant_absmax",
    "quant_rows", "gemm_bf16", "gemm_fp8", "silu", "swiglu",
    "decode_dual", "decode_down", "decode_gemv", "decode_gemv_bf16", "block_forward",
    "sigmoid", "swiglu_bwd", "rmsnorm_bwd", "transpose", "matmul_tn", "linear_bwd", "block_backward",
]
