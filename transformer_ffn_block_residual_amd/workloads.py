"""Seeded synthetic inputs for the FFN block, shared by the tests, the benchmark
and the CPU baseline.

This module holds shapes, distributions and random numbers only: none of the
block's arithmetic.  Tensors come out as host numpy arrays of bit patterns
(bf16 as uint16) so that both the device path and the CPU oracle read exactly
the same bits.

Random numbers: numpy's PCG64 seeded with ``[seed, stream]`` — one stream per
tensor — drawn in float32 and rounded to bf16 by torch's CPU conversion
(round to nearest even).

The five workloads (sizes as the block is run in a LLaMA/Qwen2-style trainer
and in a single-token decoder):

  tiny      N=64,   C=256,  H=768,   bf16, eps 1e-5, projections ~N(0, 1/sqrt(fan_in))
  decode    M=1,    C=4096, H=14336, FP8 weights with per-row scales, x ~N(0,1)
  prefill   N=4096, C=4096, H=14336, bf16, eps 1e-5
  prefill8  same shape, FP8 per-tensor; 0.1% of residual/attention inputs x50
  qwen7b8   N=8192, C=3584, H=18944, FP8 per-tensor, eps 1e-6,
            plus a 16-token decode batch over the same FP8 weights

Residual stream and attention output ~N(0,1); RMSNorm weight ~U(0.5, 1.5);
projection weights ~N(0, 0.02) except in ``tiny``.
"""

from dataclasses import dataclass

import numpy as np
import torch

STREAM_INP, STREAM_ADDEND, STREAM_WNORM, STREAM_WGU, STREAM_WD = 1, 2, 3, 4, 5
STREAM_OUTLIER_INP, STREAM_OUTLIER_ADD = 6, 7
STREAM_DEC_X, STREAM_DEC_WG, STREAM_DEC_WU, STREAM_DEC_WD = 8, 9, 10, 11


@dataclass(frozen=True)
class Workload:
    name: str
    N: int            # prefill rows (B*T); 0 for decode-only workloads
    C: int            # hidden size
    H: int            # intermediate size
    eps: float
    fp8: bool         # FP8 (per-tensor e4m3) matmuls in the prefill block
    outliers: bool    # 0.1% of the residual / attention inputs scaled x50
    decode_M: int     # decode tokens (0: no decode part)
    w_std: float      # projection weight std (None-like 0: 1/sqrt(fan_in))
    seed: int


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 768, 1e-5, False, False, 0, 0.0, 1001),
    "decode": Workload("decode", 0, 4096, 14336, 0.0, True, False, 1, 0.02, 1002),
    "prefill": Workload("prefill", 4096, 4096, 14336, 1e-5, False, False, 0, 0.02, 1003),
    "prefill8": Workload("prefill8", 4096, 4096, 14336, 1e-5, True, True, 0, 0.02, 1004),
    "qwen7b8": Workload("qwen7b8", 8192, 3584, 18944, 1e-6, True, False, 16, 0.02, 1005),
}


def _rng(seed, stream):
    return np.random.Generator(np.random.PCG64([seed, stream]))


def to_bf16_bits(x_f32):
    """float32 array -> bf16 bit patterns (uint16), torch's round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std, seed, stream):
    x = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x)


def uniform_bf16(shape, lo, hi, seed, stream):
    x = _rng(seed, stream).random(size=shape, dtype=np.float32)
    return to_bf16_bits(np.float32(lo) + x * np.float32(hi - lo))


def _with_outliers(x_f32, seed, stream, p=0.001, factor=50.0):
    mask = _rng(seed, stream).random(size=x_f32.shape) < p
    x_f32[mask] *= np.float32(factor)
    return x_f32


def block_inputs(N, C, H, seed, w_std=0.02, outliers=False):
    """Inputs of one prefill block: residual stream ``inp`` [N,C], attention
    output ``addend`` [N,C], RMSNorm weight [C], gate+up weight [2H,C]
    (gate rows first) and down weight [C,H], all bf16 bit patterns.
    w_std = 0 draws the projections with std 1/sqrt(fan_in)."""
    r_inp = _rng(seed, STREAM_INP).standard_normal(size=(N, C), dtype=np.float32)
    r_add = _rng(seed, STREAM_ADDEND).standard_normal(size=(N, C), dtype=np.float32)
    if outliers:
        r_inp = _with_outliers(r_inp, seed, STREAM_OUTLIER_INP)
        r_add = _with_outliers(r_add, seed, STREAM_OUTLIER_ADD)
    std_gu = w_std if w_std else 1.0 / np.sqrt(C)
    std_d = w_std if w_std else 1.0 / np.sqrt(H)
    return {
        "inp": to_bf16_bits(r_inp),
        "addend": to_bf16_bits(r_add),
        "w_norm": uniform_bf16((C,), 0.5, 1.5, seed, STREAM_WNORM),
        "w_gu": normal_bf16((2 * H, C), std_gu, seed, STREAM_WGU),
        "w_d": normal_bf16((C, H), std_d, seed, STREAM_WD),
    }


def decode_inputs(M, C, H, seed, w_std=0.02, with_weights=True):
    """Decode inputs: tokens ``x`` [M,C] ~N(0,1) and bf16 master weights for
    gate [H,C], up [H,C] and down [C,H] ~N(0, w_std), which each side
    quantises row by row to e4m3 before the decode runs."""
    d = {"x": normal_bf16((M, C), 1.0, seed, STREAM_DEC_X)}
    if with_weights:
        d["w_gate"] = normal_bf16((H, C), w_std, seed, STREAM_DEC_WG)
        d["w_up"] = normal_bf16((H, C), w_std, seed, STREAM_DEC_WU)
        d["w_down"] = normal_bf16((C, H), w_std, seed, STREAM_DEC_WD)
    return d


def workload_inputs(name):
    """All inputs of a named workload (host arrays)."""
    w = WORKLOADS[name]
    out = {}
    if w.N:
        out.update(block_inputs(w.N, w.C, w.H, w.seed, w.w_std, w.outliers))
    if w.decode_M:
        out["decode"] = decode_inputs(w.decode_M, w.C, w.H, w.seed, w.w_std,
                                      with_weights=(w.N == 0))
    return out
