"""The plain C++ oracle (``ffn_oracle.cpp``): loader and numpy wrappers.
TEST INFRASTRUCTURE ONLY.

Same function names and array conventions as the numpy oracle (bf16 as uint16
bit patterns, e4m3 as uint8, fp32 scalars and vectors as float32), for the
forward block and the FP8 decode.  The two are independent implementations:
the numpy oracle sums exactly (fp64) and rounds once; this one is the fp32
form with a fixed 16-way summation order and ``std::thread`` over output
rows, fast enough to check whole full-size outputs and to serve as the CPU
baseline.  ``build()`` compiles it with the host C++ compiler; ``lib()``
compiles it on first use when the library is missing or older than its
source.
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ffn_oracle.cpp")
LIB = os.path.join(HERE, "libffn_oracle.so")
CXX = os.environ.get("CXX", "g++")
# portable x86-64 with AVX2/FMA vectors; no contraction (the products are
# exact anyway) and no fast-math, so the stated order is the order computed
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "-mavx2", "-mfma", "-ffp-contract=off", "-pthread"]

_lib = None


def build():
    """Compile ffn_oracle.cpp into libffn_oracle.so next to it."""
    tmp = LIB + ".tmp"
    cmd = [CXX, *FLAGS, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P, I64, F, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        sig = {
            "ffo_bf16_round": [P, P, I64],
            "ffo_e4m3_encode": [P, P, I64],
            "ffo_e4m3_decode": [P, P, I64],
            "ffo_rmsnorm_fwd": [P, P, P, P, P, P, P, F, I64, I64, I],
            "ffo_absmax": [P, I64],
            "ffo_quant": [P, P, I64, F, I],
            "ffo_gemm_bf16": [P, P, P, I64, I64, I64, I],
            "ffo_gemm_fp8": [P, P, F, P, F, I64, I64, I64, I],
            "ffo_gemm_abs_bf16": [P, P, P, I64, I64, I64, I],
            "ffo_gemm_abs_fp8": [P, P, F, P, F, I64, I64, I64, I],
            "ffo_swiglu": [P, P, I64, I64, I],
            "ffo_decode": [P, P, P, P, P, P, P, P, P, I64, I64, I64, I],
            "ffo_cpu_info": [ctypes.c_char_p, I, ctypes.POINTER(I), ctypes.POINTER(I)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None
        L.ffo_absmax.restype = F
        L.ffo_quant.restype = F
        L.ffo_swiglu.restype = F
        _lib = L
    return _lib


def threads():
    """Threads the oracle uses: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def cpu_info():
    """(CPU model, logical CPUs, physical cores) of the host."""
    buf = ctypes.create_string_buffer(256)
    lg, ph = ctypes.c_int(0), ctypes.c_int(0)
    lib().ffo_cpu_info(buf, 256, ctypes.byref(lg), ctypes.byref(ph))
    return buf.value.decode(errors="replace"), lg.value, ph.value


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def bf16_round_f32(v):
    """float32 values -> bf16 bit patterns (round to nearest even)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().ffo_bf16_round(_p(out), _p(v), v.size)
    return out


def e4m3_encode(v):
    """float32 values -> e4m3 codes."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().ffo_e4m3_encode(_p(out), _p(v), v.size)
    return out


def e4m3_decode(q):
    q = _u8(q)
    out = np.empty(q.shape, np.float32)
    lib().ffo_e4m3_decode(_p(out), _p(q), q.size)
    return out


def rmsnorm_fwd(inp_bits, addend_bits, weight_bits, eps, nthreads=None):
    """(residual_bits or None, y_bits, rstd float32[N], absmax float32), as the
    numpy oracle's rmsnorm_fwd, in fp32."""
    inp = _u16(inp_bits)
    N, C = inp.shape
    add = None if addend_bits is None else _u16(addend_bits)
    w = _u16(weight_bits)
    y = np.empty((N, C), np.uint16)
    rstd = np.empty(N, np.float32)
    res = None if add is None else np.empty((N, C), np.uint16)
    am = np.zeros(1, np.float32)
    lib().ffo_rmsnorm_fwd(_p(y), _p(rstd), None if res is None else _p(res), _p(am), _p(inp),
                          None if add is None else _p(add), _p(w), float(eps), N, C, nthreads or threads())
    return res, y, rstd, np.float32(am[0])


def absmax_of(bits):
    x = _u16(bits)
    return np.float32(lib().ffo_absmax(_p(x), x.size))


def quant_absmax(x_bits, absmax=None, nthreads=None):
    """(codes, scale, absmax) as the numpy oracle's quant_absmax (e4m3)."""
    x = _u16(x_bits)
    if absmax is None:
        absmax = absmax_of(x)
    q = np.empty(x.shape, np.uint8)
    s = lib().ffo_quant(_p(q), _p(x), x.size, float(np.float32(absmax)), nthreads or threads())
    return q, np.float32(s), np.float32(absmax)


def gemm_bf16(x_bits, w_bits, nthreads=None):
    x, w = _u16(x_bits), _u16(w_bits)
    N, K = x.shape
    O = w.shape[0]
    out = np.empty((N, O), np.uint16)
    lib().ffo_gemm_bf16(_p(out), _p(x), _p(w), N, K, O, nthreads or threads())
    return out


def gemm_fp8(qx, sx, qw, sw, nthreads=None):
    qx, qw = _u8(qx), _u8(qw)
    N, K = qx.shape
    O = qw.shape[0]
    out = np.empty((N, O), np.uint16)
    lib().ffo_gemm_fp8(_p(out), _p(qx), float(np.float32(sx)), _p(qw), float(np.float32(sw)), N, K, O,
                       nthreads or threads())
    return out


def gemm_abs_bf16(x_bits, w_bits, nthreads=None):
    """sum_k |x[n, k]| |w[o, k]| as float32 [N, O]: the magnitude an error
    bound of the product scales with."""
    x, w = _u16(x_bits), _u16(w_bits)
    N, K = x.shape
    O = w.shape[0]
    out = np.empty((N, O), np.float32)
    lib().ffo_gemm_abs_bf16(_p(out), _p(x), _p(w), N, K, O, nthreads or threads())
    return out


def gemm_abs_fp8(qx, sx, qw, sw, nthreads=None):
    qx, qw = _u8(qx), _u8(qw)
    N, K = qx.shape
    O = qw.shape[0]
    out = np.empty((N, O), np.float32)
    lib().ffo_gemm_abs_fp8(_p(out), _p(qx), float(np.float32(sx)), _p(qw), float(np.float32(sw)), N, K, O,
                           nthreads or threads())
    return out


def swiglu(gu_bits, nthreads=None):
    gu = _u16(gu_bits)
    N, H2 = gu.shape
    h = np.empty((N, H2 // 2), np.uint16)
    am = lib().ffo_swiglu(_p(h), _p(gu), N, H2 // 2, nthreads or threads())
    return h, np.float32(am)


def decode_gemv(x_bits, wg, sg, wu, su, wd, sd, nthreads=None):
    """(y_bits [M, C], h_bits [M, H]) of the split-SiLU FP8 decode."""
    x = _u16(x_bits)
    M, C = x.shape
    wg, wu, wd = _u8(wg), _u8(wu), _u8(wd)
    H = wg.shape[0]
    sg, su, sd = (np.ascontiguousarray(v, dtype=np.float32) for v in (sg, su, sd))
    y = np.empty((M, C), np.uint16)
    h = np.empty((M, H), np.uint16)
    lib().ffo_decode(_p(y), _p(h), _p(x), _p(wg), _p(sg), _p(wu), _p(su), _p(wd), _p(sd), M, C, H,
                     nthreads or threads())
    return y, h


def block_forward(inp, addend, w_norm, w_gu, w_d, eps, fp8=False, nthreads=None):
    """One FFN block (the chain of the numpy oracle's block_forward, in fp32);
    returns the same dict of intermediates."""
    t = nthreads or threads()
    out = {}
    r, y, rstd, am_y = rmsnorm_fwd(inp, addend, w_norm, eps, t)
    r_vals = _u16(inp) if r is None else r
    out.update(residual=r, rms_input=r_vals, y=y, rstd=rstd, absmax_y=am_y)
    if not fp8:
        gu = gemm_bf16(y, w_gu, t)
        h, am_h = swiglu(gu, t)
        d = gemm_bf16(h, w_d, t)
    else:
        qw_gu, s_gu, _ = quant_absmax(w_gu, None, t)
        qw_d, s_d, _ = quant_absmax(w_d, None, t)
        qy, s_y, _ = quant_absmax(y, am_y, t)
        gu = gemm_fp8(qy, s_y, qw_gu, s_gu, t)
        h, am_h = swiglu(gu, t)
        qh, s_h, _ = quant_absmax(h, am_h, t)
        d = gemm_fp8(qh, s_h, qw_d, s_d, t)
        out.update(qw_gu=qw_gu, s_gu=s_gu, qw_d=qw_d, s_d=s_d, qy=qy, s_y=s_y, qh=qh, s_h=s_h)
    out.update(gu=gu, h=h, absmax_h=am_h, down=d)
    # closing residual: the next block's fused add, bf16(r + down) in fp32
    rv = r_vals.astype(np.uint32) << 16
    dv = d.astype(np.uint32) << 16
    out["next_residual"] = bf16_round_f32(rv.view(np.float32) + dv.view(np.float32))
    return out
