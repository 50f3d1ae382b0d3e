"""Helpers for the GPU parity tests: moving bit patterns between numpy and
device tensors, and the error measures the tests apply."""

import sys

import numpy as np
import torch

from oracle import codecs as K


def say(msg):
    """Name the case before each GPU step, flushed, so a fault names it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_u8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def dev_f32(v):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(v, np.float32)).reshape(-1)).cuda()


def host_bits(t):
    """bf16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def host_f32(t):
    return t.detach().float().cpu().numpy()


def empty_bf16(*shape):
    return torch.empty(*shape, dtype=torch.bfloat16, device="cuda")


def empty_f32(*shape):
    return torch.empty(*shape, dtype=torch.float32, device="cuda")


def empty_u8(*shape):
    return torch.empty(*shape, dtype=torch.uint8, device="cuda")


def rel_err(got_bits, ref_bits):
    """max_i |g_i - r_i| / max(|r_i|, rms(r)) over bf16 tensors: a relative
    error that falls back to the tensor's RMS where r_i is near zero."""
    g = K.bf16_bits_to_f64(got_bits).reshape(-1)
    r = K.bf16_bits_to_f64(ref_bits).reshape(-1)
    if r.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))


def ulp_diff(a_bits, b_bits):
    a = np.asarray(a_bits).astype(np.int32)
    b = np.asarray(b_bits).astype(np.int32)
    ka = np.where(a & 0x8000, -(a & 0x7FFF), a)
    kb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ka - kb)


def normwise_err(got_bits, ref_bits):
    """max_i |g_i - r_i| / max_i |r_i|: the error measured against the tensor's
    abs-max, the quantity that sets a per-tensor quantisation grid."""
    g = K.bf16_bits_to_f64(got_bits).reshape(-1)
    r = K.bf16_bits_to_f64(ref_bits).reshape(-1)
    m = np.max(np.abs(r)) if r.size else 0.0
    return float(np.max(np.abs(g - r)) / m) if m > 0 else float(np.max(np.abs(g - r), initial=0.0))


def within_dot_bound(got_bits, exact, mag, rel_out=2.0 ** -8, rel_sum=2.0 ** -14):
    """True where |g - exact| <= rel_out*|exact| + rel_sum*mag: one bf16 rounding
    of the result plus an accumulation error proportional to sum_k |a_k b_k|
    (mag).  rel_sum = 2^-14 covers fp32 accumulation over the K used in the tests
    and the f8f6f4 MFMA, whose 64-term dot products carry about 2^-16 of their
    sum of magnitudes."""
    g = K.bf16_bits_to_f64(got_bits)
    return np.abs(g - exact) <= rel_out * np.abs(exact) + rel_sum * mag


def flip_bound(dq_got, dq_ref, w_abs):
    """Sum_j |dq_got[n, j] - dq_ref[n, j]| * w_abs[o, j]: how far an output of a
    product with weights w can move when its input's dequantised values
    differ between two chains (codes that one chain rounded to a neighbouring
    grid point).  A sparse product over the differing entries, so the cost
    follows their number."""
    import scipy.sparse as sp
    d = np.abs(np.asarray(dq_got, np.float64) - np.asarray(dq_ref, np.float64))
    return np.asarray(sp.csr_matrix(d) @ np.asarray(w_abs, np.float64).T)


def rel_err_with_bound(got_bits, ref_bits, bound):
    """max_i (|g_i - r_i| - bound_i) / max(|r_i|, rms(r)): rel_err after the
    allowed movement `bound` (>= 0, the ref's shape) has been taken off."""
    g = K.bf16_bits_to_f64(got_bits)
    r = K.bf16_bits_to_f64(ref_bits)
    if r.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max((np.abs(g - r) - bound) / den))
