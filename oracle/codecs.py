"""Number formats the FFN block stores its tensors in.  TEST INFRASTRUCTURE ONLY.

* bf16 — the model dtype of every activation and of the bf16 weights
  (llmq llama_run_state.cpp, ``allocate_basic_fwd_tensors``: the LN, residual,
  SwiGLU and MLP buffers are allocated in ``Config.DType``).  Here: IEEE
  binary32 truncated to 16 bits, 1 sign, 8 exponent, 7 stored mantissa bits,
  round to nearest with ties to even.
* e4m3 — the FP8 type of the quantised matmul operands (llmq
  llama_run_state.cpp, ``allocate_fwd_quant_tensors`` allocates the quantised
  copies as ``FP8_E4M3``).  Read as the OCP E4M3FN layout: bias 7, no
  infinities, 0x7F/0xFF NaN, largest finite magnitude 448, smallest normal
  2^-6, smallest subnormal 2^-9.  Encoding rounds to nearest, ties to the even
  code, and saturates magnitudes at or above 448 to 448.
* e5m2 — the other FP8 gradient type the trainer accepts (llmq
  llama_run_state.cpp: ``use_fp8`` holds for a grad dtype of ``FP8_E4M3`` or
  ``FP8_E5M2``; the transposed gradient of ``backward_qmm`` is allocated in the
  grad dtype).  Read as the OCP E5M2 layout: bias 15, infinities at
  0x7C/0xFC, NaN above them, largest finite magnitude 57344, smallest normal
  2^-14, smallest subnormal 2^-16.  Encoding rounds to nearest, ties to the
  even code, and saturates at 57344 as the e4m3 encoder does at 448.

Each routine is written from those definitions, on whole numpy arrays, with no
bit tricks beyond reading a float32's bit pattern.
"""

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
BF16_MAX = float.fromhex("0x1.fe00000000000p+127")  # (2 - 2^-7) * 2^127


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> their exact values as float64."""
    b = np.asarray(bits).astype(np.uint16)
    f32 = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def bf16_round(v):
    """Round each value to the nearest bf16 value, ties to even.  Returns float64.

    A finite non-zero v is written as f * 2**E with 0.5 <= |f| < 1; bf16 keeps
    8 significant bits, so the rounded value is rint(f * 2**8) * 2**(E-8).
    Below the smallest normal (2^-126) the spacing is fixed at 2^-133.
    Magnitudes that round past the largest finite bf16 become infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1)
    out = np.empty_like(v)
    nan = np.isnan(v)
    f, e = np.frexp(v)
    normal = np.abs(v) >= 2.0 ** -126
    with np.errstate(over="ignore", invalid="ignore"):
        rn = np.ldexp(np.rint(np.ldexp(f, 8)), e - 8)
        rs = np.ldexp(np.rint(np.ldexp(v, 133)), -133)
    out[:] = np.where(normal, rn, rs)
    big = np.abs(out) > BF16_MAX
    out[big] = np.copysign(np.inf, v[big])
    out[np.isinf(v)] = v[np.isinf(v)]
    out[nan] = np.nan
    # rint keeps the sign of zero, so -tiny rounds to -0.0 as IEEE requires.
    return out.reshape(shape)


def f64_to_bf16_bits(v):
    """Round to bf16 (ties to even) and return the uint16 bit patterns."""
    r = bf16_round(v).reshape(-1)
    shape = np.shape(v)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(r)] = np.where(np.signbit(r[np.isnan(r)]), 0xFFC0, 0x7FC0)
    return bits.reshape(shape)


def _e4m3_table():
    codes = np.arange(256, dtype=np.uint16)
    s = (codes >> 7) & 1
    e = ((codes >> 3) & 0xF).astype(np.int64)
    m = (codes & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    val[(e == 15) & (m == 7)] = np.nan
    return val


_E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes):
    """e4m3 codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    return _E4M3_VALUES[np.asarray(codes).astype(np.uint8)]


def e4m3_encode(v):
    """Values -> e4m3 codes (uint8): round to nearest, ties to the even code,
    saturate at 448, NaN -> 0x7F with the sign bit, -0.0 -> 0x80.

    Callers that follow the kernels pass float32 values (the product that
    decides the code is taken in fp32); the encoder itself is exact for any
    float64 input.
    """
    v = np.asarray(v, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.uint8)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    code = np.zeros(a.shape, dtype=np.int64)
    # Subnormal range: the grid is 2^-9, eight steps up to the smallest normal.
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # 8 lands on code 0x08 = 2^-6
    # Normal range: a = (1 + m/8) * 2^e with e = floor(log2 a) in [-6, 8].
    nrm = ~sub
    f, ex = np.frexp(a[nrm])
    e = ex - 1
    m = np.rint((np.ldexp(a[nrm], -e) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code[nrm] = ((e + 7) << 3) | m
    out = (code.astype(np.uint8) | sign).astype(np.uint8)
    out[nan] = 0x7F | sign[nan]
    return out.reshape(shape)


def _e5m2_table():
    codes = np.arange(256, dtype=np.uint16)
    s = (codes >> 7) & 1
    e = ((codes >> 2) & 0x1F).astype(np.int64)
    m = (codes & 0x3).astype(np.float64)
    mag = np.where(e == 0, (m / 4.0) * 2.0 ** -14, (1.0 + m / 4.0) * np.power(2.0, e - 15))
    val = np.where(s == 1, -mag, mag)
    val[(e == 31) & (m == 0)] = np.where(s[(e == 31) & (m == 0)] == 1, -np.inf, np.inf)
    val[(e == 31) & (m != 0)] = np.nan
    return val


_E5M2_VALUES = _e5m2_table()


def e5m2_decode(codes):
    """e5m2 codes (uint8) -> float64 values (+-inf for 0x7C / 0xFC, NaN above)."""
    return _E5M2_VALUES[np.asarray(codes).astype(np.uint8)]


def e5m2_encode(v):
    """Values -> e5m2 codes (uint8): round to nearest, ties to the even code,
    saturate at 57344, NaN -> 0x7E with the sign bit, -0.0 -> 0x80."""
    v = np.asarray(v, dtype=np.float64)
    shape = v.shape
    v = v.reshape(-1)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.uint8)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E5M2_MAX))
    code = np.zeros(a.shape, dtype=np.int64)
    # Subnormal range: the grid is 2^-16, four steps up to the smallest normal.
    sub = a < 2.0 ** -14
    code[sub] = np.rint(a[sub] * 2.0 ** 16).astype(np.int64)  # 4 lands on code 0x04 = 2^-14
    # Normal range: a = (1 + m/4) * 2^e with e = floor(log2 a) in [-14, 15].
    nrm = ~sub
    f, ex = np.frexp(a[nrm])
    e = ex - 1
    m = np.rint((np.ldexp(a[nrm], -e) - 1.0) * 4.0).astype(np.int64)
    carry = m == 4
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    code[nrm] = ((e + 15) << 2) | m
    out = (code.astype(np.uint8) | sign).astype(np.uint8)
    out[nan] = 0x7E | sign[nan]
    return out.reshape(shape)


FP8_FORMATS = {
    "e4m3": (e4m3_encode, e4m3_decode, E4M3_MAX),
    "e5m2": (e5m2_encode, e5m2_decode, E5M2_MAX),
}
