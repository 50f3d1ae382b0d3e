"""CPU oracle for the dense SwiGLU FFN block and its FP8 decode form.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library under ``transformer_ffn_block_residual_amd/csrc`` and imports nothing
from that package.

The oracle is plain numpy.  Bit patterns cross its interface as integer
arrays (bf16 as uint16, e4m3 as uint8, fp32 as float32) so that nothing in it
depends on another library's rounding.  Reductions and dot products run in
fp64; every value the pages store (bf16 activations, fp32 rstd and scales,
e4m3 codes) is rounded exactly once to that storage type.  Where a floating
point product decides an integer code (FP8 quantisation) the product is taken
in fp32, the precision of the kernel that makes the same decision.

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
    gateup,
    down,
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
    "quant_rows", "gemm_bf16", "gemm_fp8", "silu", "swiglu", "gateup", "down",
    "decode_dual", "decode_down", "decode_gemv", "decode_gemv_bf16", "block_forward",
    "sigmoid", "swiglu_bwd", "rmsnorm_bwd", "transpose", "matmul_tn", "linear_bwd", "block_backward",
]
