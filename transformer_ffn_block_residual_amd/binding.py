"""Python binding of libffn.so: the FFN block's hot path on MI355X.

Each function has the name and argument order of its C entry point in
``include/ffn.h`` and only marshals arguments: it checks that every tensor is a
contiguous device tensor of the element type and size the call will touch
(so that no kernel is launched on a buffer that is too small), passes raw device
pointers and the stream, and turns a non-OK status into ``FFNError``.  All
arithmetic happens in the HIP kernels.  torch supplies device memory and the
stream (the current torch stream unless one is given).

There is no fallback: if the library is missing, importing this package raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libffn.so")

FFN_OK, FFN_ERR_INVALID, FFN_ERR_UNSUPPORTED, FFN_ERR_HIP = 0, 1, 2, 3
FFN_BF16, FFN_E4M3, FFN_E5M2 = 0, 1, 2
FFN_TN_ACCUMULATE, FFN_TN_TILE_GRID, FFN_TN_TILED = 1, 2, 4
_STATUS = {1: "FFN_ERR_INVALID", 2: "FFN_ERR_UNSUPPORTED", 3: "FFN_ERR_HIP"}


class FFNError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m transformer_ffn_block_residual_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sig = {
        "ffn_rmsnorm_fwd": [P, P, P, P, P, P, P, F32, I64, I64, P],
        "ffn_rmsnorm_fwd_acc": [P, P, P, P, P, P, P, F32, I64, I64, P],
        "ffn_quant_absmax_clear": [P, P, P, P, I64, P, P],
        "ffn_gateup_acc": [P, P, P, P, P, P, I32, I64, I64, I64, P],
        "ffn_quant_absmax": [P, P, P, P, I64, I32, P],
        "ffn_quant_rows": [P, P, P, I64, I64, P],
        "ffn_gateup": [P, P, P, P, P, P, I32, I32, I64, I64, I64, P],
        "ffn_gateup_swiglu_quant": [P, P, P, P, P, P, P, P, I32, I64, I64, I64, P],
        "ffn_swiglu": [P, P, P, I64, I64, P],
        "ffn_down": [P, P, P, P, P, I32, I64, I64, I64, P],
        "ffn_decode_gemv": [P, P, P, P, P, P, P, P, P, I64, I64, I64, P],
        "ffn_decode_gemv_arm": [P, P, P, P, P, P, P, P, P, P, I32, I64, I64, I64, P],
        "ffn_decode_gemv_bf16": [P, P, P, P, P, P, I64, I64, I64, P],
        "ffn_decode_pack_weight": [P, P, I64, I64, P],
        "ffn_decode_gemv_packed": [P, P, P, P, P, P, P, P, P, P, I64, I64, I64, P],
        "ffn_decode_gemv_packed_noalloc": [P, P, P, P, P, P, P, P, P, I64, I64, I64, P],
        "ffn_matmul_tn": [P, P, P, P, P, I32, I32, I64, I64, I64, P],
        "ffn_matmul_tn_swiglu_bwd": [P, P, P, P, P, P, P, I32, I32, I64, I64, I64, P],
        "ffn_transpose": [P, P, I64, I64, I64, I32, P],
        "ffn_quant_transpose": [P, P, P, P, P, I32, I64, I64, I64, P],
        "ffn_swiglu_bwd": [P, P, P, P, I64, I64, P],
        "ffn_rmsnorm_bwd": [P, P, P, P, P, P, P, P, P, I64, I64, P],
        "ffn_matmul_tn_swiglu_bwd_acc": [P, P, P, P, P, P, P, I32, I32, I64, I64, I64, P],
        "ffn_quant_transpose_clear": [P, P, P, P, P, P, I32, I64, I64, I64, P],
        "ffn_swiglu_bwd_acc": [P, P, P, P, I64, I64, P],
        "ffn_rmsnorm_bwd_acc": [P, P, P, P, P, P, P, P, P, P, I64, I64, P],
        "ffn_tile_pack": [P, P, I64, I64, P],
        "ffn_quant_absmax_clear_tiled": [P, P, P, P, I64, I64, P, P],
        "ffn_gateup_acc_tiled": [P, P, P, P, P, P, I64, I64, I64, P],
        "ffn_gateup_swiglu_quant_tiled": [P, P, P, P, P, P, P, P, I64, I64, I64, P],
        "ffn_down_tiled": [P, P, P, P, P, I64, I64, I64, P],
        "ffn_rmsnorm_fwd_tiled": [P, P, P, P, P, P, P, F32, I64, I64, P],
        "ffn_gateup_tiled_bf16": [P, P, P, P, I64, I64, I64, P],
        "ffn_down_tiled_bf16": [P, P, P, I64, I64, I64, P],
        "ffn_transpose_tiled": [P, P, I64, I64, I64, P],
        "ffn_quant_transpose_tiled": [P, P, P, P, P, P, I32, I64, I64, I64, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ffn_rmsnorm_bwd_scratch_bytes.argtypes = [I64, I64]
    lib.ffn_rmsnorm_bwd_scratch_bytes.restype = ctypes.c_int64
    lib.ffn_decode_packed_workspace_bytes.argtypes = [I64, I64, I64]
    lib.ffn_decode_packed_workspace_bytes.restype = ctypes.c_int64
    lib.ffn_tile_bytes.argtypes = [I64, I64]
    lib.ffn_tile_bytes.restype = ctypes.c_int64
    lib.ffn_decode_noalloc_scratch_bytes.argtypes = []
    lib.ffn_decode_noalloc_scratch_bytes.restype = ctypes.c_int64
    lib.ffn_last_error.restype = ctypes.c_char_p
    lib.ffn_last_error.argtypes = []
    lib.ffn_version.restype = ctypes.c_char_p
    lib.ffn_version.argtypes = []
    return lib


_lib = _load()


def version():
    return _lib.ffn_version().decode()


def last_error():
    return _lib.ffn_last_error().decode()


def _check(status):
    if status != FFN_OK:
        raise FFNError(status, last_error())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


_ELT = {torch.bfloat16: 2, torch.float32: 4, torch.uint8: 1, torch.float8_e4m3fn: 1, torch.int16: 2}


def _ptr(t, name, numel, dtypes, optional=False):
    """Device pointer of tensor t after checking it holds >= numel elements of
    one of dtypes, contiguous, on a GPU."""
    if t is None:
        if optional:
            return None
        raise FFNError(FFN_ERR_INVALID, f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise FFNError(FFN_ERR_INVALID, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise FFNError(FFN_ERR_INVALID, f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise FFNError(FFN_ERR_INVALID, f"{name}: dtype {t.dtype} not in {dtypes}")
    if numel is not None and t.numel() < numel:
        raise FFNError(FFN_ERR_INVALID, f"{name}: {t.numel()} elements < {numel} needed")
    return ctypes.c_void_p(t.data_ptr())


BF16 = (torch.bfloat16, torch.int16)
F32 = (torch.float32,)
E4M3 = (torch.uint8, torch.float8_e4m3fn)
E5M2 = (torch.uint8, torch.float8_e5m2)


def ffn_rmsnorm_fwd(y, rstd, residual_out, absmax, inp, addend, weight, eps, N, C, stream=None):
    _check(_lib.ffn_rmsnorm_fwd(
        _ptr(y, "y", N * C, BF16), _ptr(rstd, "rstd", N, F32),
        _ptr(residual_out, "residual_out", N * C, BF16, optional=True),
        _ptr(absmax, "absmax", 1, F32, optional=True),
        _ptr(inp, "inp", N * C, BF16), _ptr(addend, "addend", N * C, BF16, optional=True),
        _ptr(weight, "weight", C, BF16), float(eps), int(N), int(C), _stream(stream)))


def ffn_quant_absmax(q, scale, absmax, x, n, compute_absmax, stream=None):
    _check(_lib.ffn_quant_absmax(
        _ptr(q, "q", n, E4M3), _ptr(scale, "scale", 1, F32), _ptr(absmax, "absmax", 1, F32),
        _ptr(x, "x", n, BF16), int(n), int(bool(compute_absmax)), _stream(stream)))


def ffn_rmsnorm_fwd_acc(y, rstd, residual_out, absmax, inp, addend, weight, eps, N, C, stream=None):
    """ffn_rmsnorm_fwd max-accumulating into a caller-zeroed abs-max word."""
    _check(_lib.ffn_rmsnorm_fwd_acc(
        _ptr(y, "y", N * C, BF16), _ptr(rstd, "rstd", N, F32),
        _ptr(residual_out, "residual_out", N * C, BF16, optional=True),
        _ptr(absmax, "absmax", 1, F32),
        _ptr(inp, "inp", N * C, BF16), _ptr(addend, "addend", N * C, BF16, optional=True),
        _ptr(weight, "weight", C, BF16), float(eps), int(N), int(C), _stream(stream)))


def ffn_quant_absmax_clear(q, scale, absmax, x, n, clear, stream=None):
    """Quantise with the given abs-max and zero the abs-max word `clear`."""
    _check(_lib.ffn_quant_absmax_clear(
        _ptr(q, "q", n, E4M3), _ptr(scale, "scale", 1, F32), _ptr(absmax, "absmax", 1, F32),
        _ptr(x, "x", n, BF16), int(n), _ptr(clear, "clear", 1, F32), _stream(stream)))


def ffn_quant_rows(q, row_scale, w, rows, cols, stream=None):
    _check(_lib.ffn_quant_rows(
        _ptr(q, "q", rows * cols, E4M3), _ptr(row_scale, "row_scale", rows, F32),
        _ptr(w, "w", rows * cols, BF16), int(rows), int(cols), _stream(stream)))


def _dt_elems(dtype):
    return E4M3 if dtype == FFN_E4M3 else BF16


def ffn_gateup(out, out_absmax, x, x_scale, w, w_scale, dtype, fuse_swiglu, N, C, H, stream=None):
    fp8 = dtype == FFN_E4M3
    _check(_lib.ffn_gateup(
        _ptr(out, "out", N * (H if fuse_swiglu else 2 * H), BF16),
        _ptr(out_absmax, "out_absmax", 1, F32, optional=True),
        _ptr(x, "x", N * C, _dt_elems(dtype)), _ptr(x_scale, "x_scale", 1, F32, optional=not fp8),
        _ptr(w, "w", 2 * H * C, _dt_elems(dtype)), _ptr(w_scale, "w_scale", 1, F32, optional=not fp8),
        int(dtype), int(bool(fuse_swiglu)), int(N), int(C), int(H), _stream(stream)))


def ffn_gateup_acc(h, h_absmax, x, x_scale, w, w_scale, dtype, N, C, H, stream=None):
    """ffn_gateup with the SwiGLU epilogue, max-accumulating into a
    caller-zeroed abs-max word."""
    fp8 = dtype == FFN_E4M3
    _check(_lib.ffn_gateup_acc(
        _ptr(h, "h", N * H, BF16), _ptr(h_absmax, "h_absmax", 1, F32),
        _ptr(x, "x", N * C, _dt_elems(dtype)), _ptr(x_scale, "x_scale", 1, F32, optional=not fp8),
        _ptr(w, "w", 2 * H * C, _dt_elems(dtype)), _ptr(w_scale, "w_scale", 1, F32, optional=not fp8),
        int(dtype), int(N), int(C), int(H), _stream(stream)))


def ffn_gateup_swiglu_quant(q, q_scale, h_absmax, h_absmax_known, x, x_scale, w, w_scale, dtype, N, C, H,
                            stream=None):
    fp8 = dtype == FFN_E4M3
    _check(_lib.ffn_gateup_swiglu_quant(
        _ptr(q, "q", N * H, E4M3), _ptr(q_scale, "q_scale", 1, F32),
        _ptr(h_absmax, "h_absmax", 1, F32, optional=True), _ptr(h_absmax_known, "h_absmax_known", 1, F32),
        _ptr(x, "x", N * C, _dt_elems(dtype)), _ptr(x_scale, "x_scale", 1, F32, optional=not fp8),
        _ptr(w, "w", 2 * H * C, _dt_elems(dtype)), _ptr(w_scale, "w_scale", 1, F32, optional=not fp8),
        int(dtype), int(N), int(C), int(H), _stream(stream)))


def ffn_swiglu(h, absmax, gateup, N, H, stream=None):
    _check(_lib.ffn_swiglu(
        _ptr(h, "h", N * H, BF16), _ptr(absmax, "absmax", 1, F32, optional=True),
        _ptr(gateup, "gateup", N * 2 * H, BF16), int(N), int(H), _stream(stream)))


def ffn_down(out, h, h_scale, w, w_scale, dtype, N, H, C, stream=None):
    fp8 = dtype == FFN_E4M3
    _check(_lib.ffn_down(
        _ptr(out, "out", N * C, BF16), _ptr(h, "h", N * H, _dt_elems(dtype)),
        _ptr(h_scale, "h_scale", 1, F32, optional=not fp8),
        _ptr(w, "w", C * H, _dt_elems(dtype)), _ptr(w_scale, "w_scale", 1, F32, optional=not fp8),
        int(dtype), int(N), int(H), int(C), _stream(stream)))


def ffn_tile_bytes(rows, row_bytes):
    """Bytes of the tiled form of a [rows, row_bytes] operand (whole 64-row
    groups); raises for a row_bytes that is not a multiple of 64."""
    n = _lib.ffn_tile_bytes(int(rows), int(row_bytes))
    if n < 0:
        raise FFNError(FFN_ERR_UNSUPPORTED, f"no tiled layout for rows={rows}, row_bytes={row_bytes}")
    return n


def _tiled_numel(rows, row_bytes):
    return _lib.ffn_tile_bytes(int(rows), int(row_bytes)) if row_bytes % 64 == 0 and rows >= 0 else 0


def ffn_tile_pack(out, inp, rows, row_bytes, stream=None):
    """Tiled copy of a row-major [rows, row_bytes] byte operand."""
    _check(_lib.ffn_tile_pack(
        _ptr(out, "out", _tiled_numel(rows, row_bytes), E4M3), _ptr(inp, "in", rows * row_bytes, E4M3),
        int(rows), int(row_bytes), _stream(stream)))


def ffn_quant_absmax_clear_tiled(q, scale, absmax, x, rows, cols, clear, stream=None):
    """ffn_quant_absmax_clear with the codes of [rows, cols] stored tiled;
    clear may be None."""
    _check(_lib.ffn_quant_absmax_clear_tiled(
        _ptr(q, "q", _tiled_numel(rows, cols), E4M3), _ptr(scale, "scale", 1, F32),
        _ptr(absmax, "absmax", 1, F32), _ptr(x, "x", rows * cols, BF16), int(rows), int(cols),
        _ptr(clear, "clear", 1, F32, optional=True), _stream(stream)))


def ffn_gateup_acc_tiled(h, h_absmax, x, x_scale, w, w_scale, N, C, H, stream=None):
    """ffn_gateup_acc (e4m3) on tiled x and w."""
    _check(_lib.ffn_gateup_acc_tiled(
        _ptr(h, "h", N * H, BF16), _ptr(h_absmax, "h_absmax", 1, F32),
        _ptr(x, "x", _tiled_numel(N, C), E4M3), _ptr(x_scale, "x_scale", 1, F32),
        _ptr(w, "w", _tiled_numel(2 * H, C), E4M3), _ptr(w_scale, "w_scale", 1, F32),
        int(N), int(C), int(H), _stream(stream)))


def ffn_gateup_swiglu_quant_tiled(q, q_scale, h_absmax, h_absmax_known, x, x_scale, w, w_scale, N, C, H,
                                  stream=None):
    """ffn_gateup_swiglu_quant (e4m3) on tiled x and w, storing tiled codes."""
    _check(_lib.ffn_gateup_swiglu_quant_tiled(
        _ptr(q, "q", _tiled_numel(N, H), E4M3), _ptr(q_scale, "q_scale", 1, F32),
        _ptr(h_absmax, "h_absmax", 1, F32, optional=True), _ptr(h_absmax_known, "h_absmax_known", 1, F32),
        _ptr(x, "x", _tiled_numel(N, C), E4M3), _ptr(x_scale, "x_scale", 1, F32),
        _ptr(w, "w", _tiled_numel(2 * H, C), E4M3), _ptr(w_scale, "w_scale", 1, F32),
        int(N), int(C), int(H), _stream(stream)))


def ffn_down_tiled(out, h, h_scale, w, w_scale, N, H, C, stream=None):
    """ffn_down (e4m3) on tiled h and w."""
    _check(_lib.ffn_down_tiled(
        _ptr(out, "out", N * C, BF16), _ptr(h, "h", _tiled_numel(N, H), E4M3), _ptr(h_scale, "h_scale", 1, F32),
        _ptr(w, "w", _tiled_numel(C, H), E4M3), _ptr(w_scale, "w_scale", 1, F32),
        int(N), int(H), int(C), _stream(stream)))


def ffn_rmsnorm_fwd_tiled(y, rstd, residual_out, absmax, inp, addend, weight, eps, N, C, stream=None):
    """ffn_rmsnorm_fwd with y stored tiled (rows of 2C bytes)."""
    _check(_lib.ffn_rmsnorm_fwd_tiled(
        _ptr(y, "y", _tiled_numel(N, 2 * C) // 2, BF16), _ptr(rstd, "rstd", N, F32),
        _ptr(residual_out, "residual_out", N * C, BF16, optional=True),
        _ptr(absmax, "absmax", 1, F32, optional=True),
        _ptr(inp, "inp", N * C, BF16), _ptr(addend, "addend", N * C, BF16, optional=True),
        _ptr(weight, "weight", C, BF16), float(eps), int(N), int(C), _stream(stream)))


def ffn_gateup_tiled_bf16(h, h_absmax, x, w, N, C, H, stream=None):
    """bf16 gate+up with the SwiGLU epilogue on tiled x and w, h stored tiled."""
    _check(_lib.ffn_gateup_tiled_bf16(
        _ptr(h, "h", _tiled_numel(N, 2 * H) // 2, BF16), _ptr(h_absmax, "h_absmax", 1, F32, optional=True),
        _ptr(x, "x", _tiled_numel(N, 2 * C) // 2, BF16), _ptr(w, "w", _tiled_numel(2 * H, 2 * C) // 2, BF16),
        int(N), int(C), int(H), _stream(stream)))


def ffn_down_tiled_bf16(out, h, w, N, H, C, stream=None):
    """bf16 down projection on tiled h and w."""
    _check(_lib.ffn_down_tiled_bf16(
        _ptr(out, "out", N * C, BF16), _ptr(h, "h", _tiled_numel(N, 2 * H) // 2, BF16),
        _ptr(w, "w", _tiled_numel(C, 2 * H) // 2, BF16), int(N), int(H), int(C), _stream(stream)))


def _decode_gemv_args(out, h, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream):
    return (_ptr(out, "out", M * C, BF16), _ptr(h, "h", M * H, BF16), _ptr(x, "x", M * C, BF16),
            _ptr(w_gate, "w_gate", H * C, E4M3), _ptr(s_gate, "s_gate", H, F32),
            _ptr(w_up, "w_up", H * C, E4M3), _ptr(s_up, "s_up", H, F32),
            _ptr(w_down, "w_down", C * H, E4M3), _ptr(s_down, "s_down", C, F32),
            int(M), int(C), int(H), _stream(stream))


def ffn_decode_gemv(out, h, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream=None):
    _check(_lib.ffn_decode_gemv(*_decode_gemv_args(out, h, x, w_gate, s_gate, w_up, s_up, w_down, s_down,
                                                   M, C, H, stream)))


FFN_DECODE_SPLIT_SILU, FFN_DECODE_SILU_INPUT, FFN_DECODE_PER_PROJECTION = 0, 1, 2


def _decode_arm_args(out, h, gu, x, w_gate, s_gate, w_up, s_up, w_down, s_down, arm, M, C, H, stream):
    split = arm == FFN_DECODE_SPLIT_SILU
    return (_ptr(out, "out", M * C, BF16), _ptr(h, "h", M * H, BF16),
            _ptr(gu, "gu", M * 2 * H, BF16, optional=split), _ptr(x, "x", M * C, BF16),
            _ptr(w_gate, "w_gate", H * C, E4M3), _ptr(s_gate, "s_gate", H, F32),
            _ptr(w_up, "w_up", H * C, E4M3), _ptr(s_up, "s_up", H, F32),
            _ptr(w_down, "w_down", C * H, E4M3), _ptr(s_down, "s_down", C, F32),
            int(arm), int(M), int(C), int(H), _stream(stream))


def ffn_decode_gemv_arm(out, h, gu, x, w_gate, s_gate, w_up, s_up, w_down, s_down, arm, M, C, H, stream=None):
    _check(_lib.ffn_decode_gemv_arm(*_decode_arm_args(out, h, gu, x, w_gate, s_gate, w_up, s_up, w_down, s_down,
                                                      arm, M, C, H, stream)))


def _decode_bf16_args(out, h, x, w_gate, w_up, w_down, M, C, H, stream):
    return (_ptr(out, "out", M * C, BF16), _ptr(h, "h", M * H, BF16), _ptr(x, "x", M * C, BF16),
            _ptr(w_gate, "w_gate", H * C, BF16), _ptr(w_up, "w_up", H * C, BF16),
            _ptr(w_down, "w_down", C * H, BF16), int(M), int(C), int(H), _stream(stream))


def ffn_decode_gemv_bf16(out, h, x, w_gate, w_up, w_down, M, C, H, stream=None):
    _check(_lib.ffn_decode_gemv_bf16(*_decode_bf16_args(out, h, x, w_gate, w_up, w_down, M, C, H, stream)))


def _bound(fn, args):
    def call():
        _check(fn(*args))
    return call


def bind_decode_gemv(out, h, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream=None):
    """ffn_decode_gemv with its arguments checked and marshalled once: returns
    a no-argument callable that issues the same call (same tensors, sizes and
    stream) again.  For per-token loops where the checks would cost more host
    time than the GPU spends on the call; the tensors must stay alive."""
    return _bound(_lib.ffn_decode_gemv,
                  _decode_gemv_args(out, h, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream))


def bind_decode_gemv_arm(out, h, gu, x, w_gate, s_gate, w_up, s_up, w_down, s_down, arm, M, C, H, stream=None):
    """ffn_decode_gemv_arm bound once, as bind_decode_gemv."""
    return _bound(_lib.ffn_decode_gemv_arm,
                  _decode_arm_args(out, h, gu, x, w_gate, s_gate, w_up, s_up, w_down, s_down, arm, M, C, H, stream))


def bind_decode_gemv_bf16(out, h, x, w_gate, w_up, w_down, M, C, H, stream=None):
    """ffn_decode_gemv_bf16 bound once, as bind_decode_gemv."""
    return _bound(_lib.ffn_decode_gemv_bf16, _decode_bf16_args(out, h, x, w_gate, w_up, w_down, M, C, H, stream))


def ffn_decode_pack_weight(packed, w, rows, cols, stream=None):
    _check(_lib.ffn_decode_pack_weight(
        _ptr(packed, "packed", rows * cols, E4M3), _ptr(w, "w", rows * cols, E4M3), int(rows), int(cols),
        _stream(stream)))


def ffn_decode_packed_workspace_bytes(M, C, H):
    return int(_lib.ffn_decode_packed_workspace_bytes(int(M), int(C), int(H)))


def _decode_packed_args(out, h, ws, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream):
    need = ffn_decode_packed_workspace_bytes(M, C, H)
    return (_ptr(out, "out", M * C, BF16), _ptr(h, "h", M * H, BF16),
            _ptr(ws, "workspace", max(need, 0) // 2, BF16), _ptr(x, "x", M * C, BF16),
            _ptr(w_gate, "w_gate", H * C, E4M3), _ptr(s_gate, "s_gate", H, F32),
            _ptr(w_up, "w_up", H * C, E4M3), _ptr(s_up, "s_up", H, F32),
            _ptr(w_down, "w_down", C * H, E4M3), _ptr(s_down, "s_down", C, F32),
            int(M), int(C), int(H), _stream(stream))


def ffn_decode_gemv_packed(out, h, ws, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream=None):
    """ffn_decode_gemv on packed weights (ffn_decode_pack_weight); ws: a bf16
    tensor of at least ffn_decode_packed_workspace_bytes(M, C, H) bytes."""
    _check(_lib.ffn_decode_gemv_packed(*_decode_packed_args(out, h, ws, x, w_gate, s_gate, w_up, s_up, w_down,
                                                            s_down, M, C, H, stream)))


def bind_decode_gemv_packed(out, h, ws, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream=None):
    """ffn_decode_gemv_packed bound once, as bind_decode_gemv."""
    return _bound(_lib.ffn_decode_gemv_packed,
                  _decode_packed_args(out, h, ws, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream))


def ffn_decode_noalloc_scratch_bytes():
    return int(_lib.ffn_decode_noalloc_scratch_bytes())


def ffn_decode_gemv_packed_noalloc(out, h, x, w_gate, s_gate, w_up, s_up, w_down, s_down, M, C, H, stream=None):
    """ffn_decode_gemv_packed with the library's built-in device scratch as
    its workspace: no buffer beyond the inputs and outputs."""
    _check(_lib.ffn_decode_gemv_packed_noalloc(
        _ptr(out, "out", M * C, BF16), _ptr(h, "h", M * H, BF16), _ptr(x, "x", M * C, BF16),
        _ptr(w_gate, "w_gate", H * C, E4M3), _ptr(s_gate, "s_gate", H, F32),
        _ptr(w_up, "w_up", H * C, E4M3), _ptr(s_up, "s_up", H, F32),
        _ptr(w_down, "w_down", C * H, E4M3), _ptr(s_down, "s_down", C, F32),
        int(M), int(C), int(H), _stream(stream)))


# ----------------------------------------------------------------------------- backward

def ffn_matmul_tn(out, a, a_scale, b, b_scale, dtype, flags, M, N, K, stream=None):
    """dtype FFN_BF16 / FFN_E4M3: both operands in it; FFN_E5M2: a holds e5m2
    codes (the gradient), b e4m3 codes.  flags: FFN_TN_ACCUMULATE (or True),
    FFN_TN_TILE_GRID and/or FFN_TN_TILED (tiled FP8 operands)."""
    fp8 = dtype in (FFN_E4M3, FFN_E5M2)
    a_dt = E5M2 if dtype == FFN_E5M2 else _dt_elems(dtype)
    b_dt = E4M3 if fp8 else BF16
    tl = int(flags) & FFN_TN_TILED
    _check(_lib.ffn_matmul_tn(
        _ptr(out, "out", M * N, BF16), _ptr(a, "a", _tiled_numel(M, K) if tl else M * K, a_dt),
        _ptr(a_scale, "a_scale", 1, F32, optional=not fp8), _ptr(b, "b", _tiled_numel(N, K) if tl else N * K, b_dt),
        _ptr(b_scale, "b_scale", 1, F32, optional=not fp8), int(dtype), int(flags),
        int(M), int(N), int(K), _stream(stream)))


def _matmul_tn_swiglu_bwd(fn, dgu, absmax, a, a_scale, b, b_scale, gu, dtype, M, H, K, stream, flags, acc):
    fp8 = dtype in (FFN_E4M3, FFN_E5M2)
    a_dt = E5M2 if dtype == FFN_E5M2 else _dt_elems(dtype)
    b_dt = E4M3 if fp8 else BF16
    tl = int(flags) & FFN_TN_TILED
    _check(fn(
        _ptr(dgu, "dgu", M * 2 * H, BF16), _ptr(absmax, "absmax", 1, F32, optional=not acc),
        _ptr(a, "a", _tiled_numel(M, K) if tl else M * K, a_dt), _ptr(a_scale, "a_scale", 1, F32, optional=not fp8),
        _ptr(b, "b", _tiled_numel(H, K) if tl else H * K, b_dt), _ptr(b_scale, "b_scale", 1, F32, optional=not fp8),
        _ptr(gu, "gu", M * 2 * H, BF16), int(dtype), int(flags), int(M), int(H), int(K), _stream(stream)))


def ffn_matmul_tn_swiglu_bwd(dgu, absmax, a, a_scale, b, b_scale, gu, dtype, M, H, K, stream=None, flags=0):
    """dgu = SwiGLU backward of gu with dh = a b^T (never stored); dtype as
    ffn_matmul_tn; flags 0, FFN_TN_TILE_GRID and/or FFN_TN_TILED.  dgu may be gu."""
    _matmul_tn_swiglu_bwd(_lib.ffn_matmul_tn_swiglu_bwd, dgu, absmax, a, a_scale, b, b_scale, gu, dtype, M, H, K,
                          stream, flags, False)


def ffn_matmul_tn_swiglu_bwd_acc(dgu, absmax, a, a_scale, b, b_scale, gu, dtype, M, H, K, stream=None, flags=0):
    """ffn_matmul_tn_swiglu_bwd, max-accumulating into a caller-zeroed absmax."""
    _matmul_tn_swiglu_bwd(_lib.ffn_matmul_tn_swiglu_bwd_acc, dgu, absmax, a, a_scale, b, b_scale, gu, dtype, M, H,
                          K, stream, flags, True)


def ffn_transpose(out, inp, rows, cols, ld_out, elt_bytes, stream=None):
    dt = BF16 if elt_bytes == 2 else E4M3
    _check(_lib.ffn_transpose(
        _ptr(out, "out", cols * ld_out, dt), _ptr(inp, "in", rows * cols, dt), int(rows), int(cols), int(ld_out),
        int(elt_bytes), _stream(stream)))


def ffn_quant_transpose(q_t, q, scale, x, absmax, rows, cols, ld_out, stream=None, code_dtype=FFN_E4M3):
    """code_dtype: FFN_E4M3 (default) or FFN_E5M2, the format of q_t and q."""
    dt = E5M2 if code_dtype == FFN_E5M2 else E4M3
    _check(_lib.ffn_quant_transpose(
        _ptr(q_t, "q_t", cols * ld_out, dt), _ptr(q, "q", rows * cols, dt, optional=True),
        _ptr(scale, "scale", 1, F32), _ptr(x, "x", rows * cols, BF16),
        _ptr(absmax, "absmax", 1, F32), int(code_dtype), int(rows), int(cols), int(ld_out), _stream(stream)))


def ffn_quant_transpose_clear(q_t, q, scale, x, absmax, clear, rows, cols, ld_out, stream=None,
                              code_dtype=FFN_E4M3):
    """ffn_quant_transpose that also zeroes the abs-max word `clear`."""
    dt = E5M2 if code_dtype == FFN_E5M2 else E4M3
    _check(_lib.ffn_quant_transpose_clear(
        _ptr(q_t, "q_t", cols * ld_out, dt), _ptr(q, "q", rows * cols, dt, optional=True),
        _ptr(scale, "scale", 1, F32), _ptr(x, "x", rows * cols, BF16),
        _ptr(absmax, "absmax", 1, F32), _ptr(clear, "clear", 1, F32), int(code_dtype), int(rows), int(cols),
        int(ld_out), _stream(stream)))


def ffn_transpose_tiled(out, inp, rows, cols, ld_out, stream=None):
    """ffn_transpose of e4m3 codes with out [cols, ld_out] stored tiled."""
    _check(_lib.ffn_transpose_tiled(
        _ptr(out, "out", _tiled_numel(cols, ld_out), E4M3), _ptr(inp, "in", rows * cols, E4M3), int(rows),
        int(cols), int(ld_out), _stream(stream)))


def ffn_quant_transpose_tiled(q_t, q, scale, x, absmax, clear, rows, cols, ld_out, stream=None,
                              code_dtype=FFN_E4M3):
    """ffn_quant_transpose(_clear) with q_t and q stored tiled; clear may be None."""
    dt = E5M2 if code_dtype == FFN_E5M2 else E4M3
    _check(_lib.ffn_quant_transpose_tiled(
        _ptr(q_t, "q_t", _tiled_numel(cols, ld_out), dt), _ptr(q, "q", _tiled_numel(rows, cols), dt, optional=True),
        _ptr(scale, "scale", 1, F32), _ptr(x, "x", rows * cols, BF16), _ptr(absmax, "absmax", 1, F32),
        _ptr(clear, "clear", 1, F32, optional=True), int(code_dtype), int(rows), int(cols), int(ld_out),
        _stream(stream)))


def ffn_swiglu_bwd(dgu, absmax, dh, gu, N, H, stream=None):
    _check(_lib.ffn_swiglu_bwd(
        _ptr(dgu, "dgu", N * 2 * H, BF16), _ptr(absmax, "absmax", 1, F32, optional=True),
        _ptr(dh, "dh", N * H, BF16), _ptr(gu, "gu", N * 2 * H, BF16), int(N), int(H), _stream(stream)))


def ffn_swiglu_bwd_acc(dgu, absmax, dh, gu, N, H, stream=None):
    """ffn_swiglu_bwd, max-accumulating into a caller-zeroed absmax."""
    _check(_lib.ffn_swiglu_bwd_acc(
        _ptr(dgu, "dgu", N * 2 * H, BF16), _ptr(absmax, "absmax", 1, F32),
        _ptr(dh, "dh", N * H, BF16), _ptr(gu, "gu", N * 2 * H, BF16), int(N), int(H), _stream(stream)))


def ffn_rmsnorm_bwd_scratch_bytes(N, C):
    return int(_lib.ffn_rmsnorm_bwd_scratch_bytes(int(N), int(C)))


def _rmsnorm_bwd_args(dinp, dweight, scratch, dresidual, dy, r, weight, rstd, N, C):
    need = ffn_rmsnorm_bwd_scratch_bytes(N, C)
    return (_ptr(dinp, "dinp", N * C, BF16), _ptr(dweight, "dweight", C, F32),
            _ptr(scratch, "scratch", max(need, 0) // 4, F32), _ptr(dresidual, "dresidual", N * C, BF16),
            _ptr(dy, "dy", N * C, BF16), _ptr(r, "r", N * C, BF16), _ptr(weight, "weight", C, BF16),
            _ptr(rstd, "rstd", N, F32))


def ffn_rmsnorm_bwd(dinp, dweight, scratch, dresidual, dy, r, weight, rstd, absmax, N, C, stream=None):
    _check(_lib.ffn_rmsnorm_bwd(
        *_rmsnorm_bwd_args(dinp, dweight, scratch, dresidual, dy, r, weight, rstd, N, C),
        _ptr(absmax, "absmax", 1, F32, optional=True), int(N), int(C), _stream(stream)))


def ffn_rmsnorm_bwd_acc(dinp, dweight, scratch, dresidual, dy, r, weight, rstd, absmax, clear, N, C, stream=None):
    """ffn_rmsnorm_bwd, max-accumulating into a caller-zeroed absmax and
    zeroing the abs-max word `clear` (nullable)."""
    _check(_lib.ffn_rmsnorm_bwd_acc(
        *_rmsnorm_bwd_args(dinp, dweight, scratch, dresidual, dy, r, weight, rstd, N, C),
        _ptr(absmax, "absmax", 1, F32), _ptr(clear, "clear", 1, F32, optional=True), int(N), int(C),
        _stream(stream)))


__all__ = [
    "ffn_rmsnorm_fwd", "ffn_rmsnorm_fwd_acc", "ffn_quant_absmax_clear", "ffn_gateup_acc", "ffn_quant_absmax", "ffn_quant_rows", "ffn_gateup", "ffn_gateup_swiglu_quant",
    "ffn_swiglu", "ffn_down", "ffn_decode_gemv", "ffn_decode_gemv_arm", "ffn_decode_gemv_bf16", "bind_decode_gemv",
    "bind_decode_gemv_arm", "bind_decode_gemv_bf16", "ffn_decode_pack_weight", "ffn_decode_packed_workspace_bytes",
    "ffn_decode_noalloc_scratch_bytes", "ffn_decode_gemv_packed_noalloc",
    "ffn_decode_gemv_packed", "bind_decode_gemv_packed",
    "ffn_matmul_tn", "ffn_matmul_tn_swiglu_bwd", "ffn_transpose", "ffn_quant_transpose", "ffn_swiglu_bwd", "ffn_rmsnorm_bwd",
    "ffn_matmul_tn_swiglu_bwd_acc", "ffn_quant_transpose_clear", "ffn_swiglu_bwd_acc", "ffn_rmsnorm_bwd_acc",
    "ffn_rmsnorm_bwd_scratch_bytes",
    "ffn_tile_bytes", "ffn_tile_pack", "ffn_quant_absmax_clear_tiled", "ffn_gateup_acc_tiled",
    "ffn_gateup_swiglu_quant_tiled", "ffn_down_tiled", "ffn_rmsnorm_fwd_tiled", "ffn_gateup_tiled_bf16",
    "ffn_down_tiled_bf16", "ffn_transpose_tiled", "ffn_quant_transpose_tiled", "FFN_TN_TILED",
    "FFN_DECODE_SPLIT_SILU", "FFN_DECODE_SILU_INPUT", "FFN_DECODE_PER_PROJECTION", "FFNError", "FFN_BF16", "FFN_E4M3", "FFN_E5M2", "FFN_TN_ACCUMULATE", "FFN_TN_TILE_GRID", "version", "last_error", "LIB_PATH",
]
