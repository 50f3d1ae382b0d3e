"""The C ABI without a GPU: libffn.so loads, exports every entry point that
include/ffn.h declares, and rejects bad arguments before touching HIP.

Every call below is built to fail validation (NULL, negative, unsupported or
misaligned arguments), so no kernel is ever launched; the fake addresses are
never dereferenced.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffn.h")
LIB = os.path.join(ROOT, "transformer_ffn_block_residual_amd", "libffn.so")

INVALID, UNSUPPORTED = 1, 2
A = 0x10000          # aligned fake device address (never dereferenced)
MIS = 0x10004        # misaligned fake address


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ffn_status_t|const char\*|int64_t)\s+(ffn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libffn.so not built (run __graft_entry__.build())")
    from transformer_ffn_block_residual_amd import binding
    return binding._lib


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["ffn_rmsnorm_fwd", "ffn_rmsnorm_fwd_acc", "ffn_quant_absmax", "ffn_quant_absmax_clear",
              "ffn_quant_rows", "ffn_gateup", "ffn_gateup_acc", "ffn_gateup_swiglu_quant",
              "ffn_swiglu", "ffn_down", "ffn_decode_gemv", "ffn_decode_gemv_arm", "ffn_decode_gemv_bf16",
              "ffn_decode_pack_weight", "ffn_decode_packed_workspace_bytes", "ffn_decode_gemv_packed",
              "ffn_matmul_tn", "ffn_matmul_tn_swiglu_bwd", "ffn_transpose", "ffn_quant_transpose", "ffn_swiglu_bwd", "ffn_rmsnorm_bwd",
              "ffn_rmsnorm_bwd_scratch_bytes", "ffn_last_error", "ffn_version", "ffn_matmul_tn_swiglu_bwd_acc",
              "ffn_quant_transpose_clear", "ffn_swiglu_bwd_acc", "ffn_rmsnorm_bwd_acc", "ffn_tile_bytes",
              "ffn_tile_pack", "ffn_quant_absmax_clear_tiled", "ffn_gateup_acc_tiled",
              "ffn_gateup_swiglu_quant_tiled", "ffn_down_tiled", "ffn_rmsnorm_fwd_tiled", "ffn_gateup_tiled_bf16",
              "ffn_down_tiled_bf16", "ffn_transpose_tiled", "ffn_quant_transpose_tiled"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.ffn_version()


def _err(lib):
    return lib.ffn_last_error().decode()


def test_rmsnorm_validation(lib):
    f = lib.ffn_rmsnorm_fwd
    assert f(None, A, A, A, A, A, A, 1e-5, 4, 256, None) == INVALID
    assert "y is NULL" in _err(lib)
    assert f(A, A, A, A, A, A, A, 1e-5, -1, 256, None) == INVALID
    assert f(A, A, None, A, A, A, A, 1e-5, 4, 256, None) == INVALID      # addend without residual_out
    assert f(A, A, A, A, A, None, A, 1e-5, 4, 256, None) == INVALID      # residual_out without addend
    assert f(A, A, A, A, A, A, A, -1.0, 4, 256, None) == INVALID
    assert f(A, A, A, A, A, A, A, 1e-5, 4, 12, None) == UNSUPPORTED      # C % 8
    assert f(A, A, A, A, A, A, A, 1e-5, 4, 32768, None) == UNSUPPORTED   # C too large
    assert f(MIS, A, A, A, A, A, A, 1e-5, 4, 256, None) == UNSUPPORTED
    assert "aligned" in _err(lib)


def test_quant_validation(lib):
    f = lib.ffn_quant_absmax
    assert f(A, A, None, A, 16, 1, None) == INVALID
    assert f(A, A, A, A, -3, 1, None) == INVALID
    assert f(A, A + 64, A + 64, A, 16, 0, None) == INVALID  # scale aliases absmax
    assert f(MIS, A, A + 64, A, 16, 0, None) == UNSUPPORTED
    g = lib.ffn_quant_rows
    assert g(A, A, A, 4, 12, None) == UNSUPPORTED
    assert g(A, None, A, 4, 16, None) == INVALID


def test_absmax_accumulating_forms_validation(lib):
    """The forms that accumulate into a caller-zeroed abs-max word, and the
    quantiser that reads one word and zeroes another."""
    f = lib.ffn_rmsnorm_fwd_acc
    assert f(A, A, None, None, A, None, A, 1e-5, 4, 256, None) == INVALID        # no abs-max word
    assert "absmax is NULL" in _err(lib)
    assert f(None, A, None, A, A, None, A, 1e-5, 4, 256, None) == INVALID
    assert "ffn_rmsnorm_fwd_acc: y is NULL" in _err(lib)
    assert f(A, A, None, A, A, None, A, 1e-5, 4, 12, None) == UNSUPPORTED
    q = lib.ffn_quant_absmax_clear          # q, scale, absmax, x, n, clear
    B, C_, D = 0x20000, 0x30000, 0x40000
    assert q(A, B, C_, A, 16, None, None) == INVALID                             # no word to clear
    assert q(A, B, C_, A, 16, C_, None) == INVALID                               # clear aliases absmax
    assert q(A, B, C_, A, 16, B, None) == INVALID                                # clear aliases scale
    assert q(A, C_, C_, A, 16, D, None) == INVALID                               # scale aliases absmax
    assert "three words" in _err(lib)
    assert q(A, B, C_, A, -1, D, None) == INVALID
    assert q(MIS, B, C_, A, 16, D, None) == UNSUPPORTED
    g = lib.ffn_gateup_acc                  # h, h_absmax, x, xs, w, ws, dtype, N, C, H
    assert g(A, None, A, None, A, None, 0, 64, 256, 768, None) == INVALID         # no abs-max word
    assert g(A, B, A, None, A, None, 1, 64, 256, 768, None) == INVALID            # fp8 without scales
    assert g(A, B, A, B, A, C_, 1, 64, 256, 768, None) == INVALID                 # abs-max aliases x_scale
    assert "alias" in _err(lib)
    assert g(A, B, A, None, A, None, 0, 64, 256, 100, None) == UNSUPPORTED        # H % 128
    assert g(A, B, A, None, A, None, 0, 64, 200, 768, None) == UNSUPPORTED        # C % 128
    assert g(MIS, B, A, None, A, None, 0, 64, 256, 768, None) == UNSUPPORTED


def test_gemm_validation(lib):
    f = lib.ffn_gateup
    assert f(A, None, A, None, A, None, 1, 1, 64, 256, 768, None) == INVALID   # fp8 without scales
    assert f(A, None, A, A, A, A, 7, 1, 64, 256, 768, None) == INVALID         # unknown dtype
    assert f(A, None, A, A, A, A, 2, 1, 64, 256, 768, None) == INVALID         # e5m2: gradients only
    assert f(A, None, A, None, A, None, 0, 1, 64, 200, 768, None) == UNSUPPORTED  # C % 128
    assert f(A, None, A, None, A, None, 0, 1, 64, 256, 100, None) == UNSUPPORTED  # H % 128
    assert f(A, None, A, None, A, None, 0, 1, -64, 256, 768, None) == INVALID
    assert f(A, None, MIS, None, A, None, 0, 1, 64, 256, 768, None) == UNSUPPORTED
    assert f(A, None, A, None, A, None, 0, 1, 1 << 20, 4096, 768, None) == UNSUPPORTED  # > 4 GiB operand
    E, S2 = 0x90000, 0xA0000
    assert f(A, E, A, E, A, S2, 1, 1, 64, 256, 768, None) == INVALID           # abs-max aliases x_scale
    assert f(A, S2, A, E, A, S2, 1, 1, 64, 256, 768, None) == INVALID          # abs-max aliases w_scale
    assert "alias" in _err(lib)
    g = lib.ffn_gateup_swiglu_quant   # q, q_scale, h_absmax, h_absmax_known, x, xs, w, ws, dtype, N, C, H
    B, C_, D = 0x20000, 0x30000, 0x40000
    assert g(A, B, C_, None, A, None, A, None, 0, 64, 256, 768, None) == INVALID      # no known abs-max
    assert "h_absmax_known is NULL" in _err(lib)
    assert g(A, B, C_, C_, A, None, A, None, 0, 64, 256, 768, None) == INVALID        # known aliases h_absmax
    assert g(A, B, C_, B, A, None, A, None, 0, 64, 256, 768, None) == INVALID         # known aliases q_scale
    assert "alias" in _err(lib)
    assert g(A, B, C_, D, A, None, A, None, 1, 64, 256, 768, None) == INVALID         # fp8 without scales
    assert g(A, B, C_, D, A, None, A, None, 0, 64, 256, 100, None) == UNSUPPORTED     # H % 128
    assert g(MIS, B, C_, D, A, None, A, None, 0, 64, 256, 768, None) == UNSUPPORTED   # misaligned q
    assert g(A, None, C_, D, A, None, A, None, 0, 64, 256, 768, None) == INVALID      # no q_scale
    assert g(A, B, C_, D, A, C_, A, 0x50000, 1, 64, 256, 768, None) == INVALID        # h_absmax aliases x_scale
    assert g(A, B, C_, D, A, 0x50000, A, B, 1, 64, 256, 768, None) == INVALID         # q_scale aliases w_scale
    d = lib.ffn_down
    assert d(A, A, None, A, None, 1, 64, 768, 256, None) == INVALID
    assert d(A, A, None, A, None, 0, 64, 700, 256, None) == UNSUPPORTED
    assert d(None, A, None, A, None, 0, 64, 768, 256, None) == INVALID
    s = lib.ffn_swiglu
    assert s(A, None, A, 4, 12, None) == UNSUPPORTED
    assert s(None, None, A, 4, 16, None) == INVALID


def test_tiled_layout_validation(lib):
    tb = lib.ffn_tile_bytes
    assert tb(1, 64) == 64 * 64 and tb(64, 128) == 64 * 128 and tb(65, 128) == 128 * 128 and tb(0, 64) == 0
    assert tb(10, 100) == -1 and tb(-1, 64) == -1
    p = lib.ffn_tile_pack                       # out, in, rows, row_bytes
    assert p(None, A, 64, 128, None) == INVALID
    assert p(A, A, 64, 100, None) == UNSUPPORTED          # row_bytes % 64
    assert p(A, A, -1, 128, None) == INVALID
    assert p(MIS, 0x900000, 64, 128, None) == UNSUPPORTED
    assert p(A, A + 64, 64, 128, None) == INVALID          # out overlaps in
    assert "overlaps" in _err(lib)
    assert p(A, 0x900000, 0, 128, None) == 0              # no rows: nothing to launch, no HIP call
    q = lib.ffn_quant_absmax_clear_tiled       # q, scale, absmax, x, rows, cols, clear
    S, M, Z = 0x20000, 0x30000, 0x40000
    assert q(A, S, S, A, 64, 256, Z, None) == INVALID      # scale aliases absmax
    assert q(A, S, M, A, 64, 256, M, None) == INVALID      # clear aliases absmax
    assert q(A, S, M, A, 64, 256, S, None) == INVALID      # clear aliases scale
    assert q(A, S, M, A, 64, 192, Z, None) == UNSUPPORTED  # cols % 128
    assert q(A, S, M, A, -2, 256, None, None) == INVALID
    assert q(A, S, M, 0x900004, 64, 256, None, None) == UNSUPPORTED     # misaligned x
    assert q(None, S, M, A, 64, 256, None, None) == INVALID
    assert q(0x100000 + 1024, S, M, 0x100000, 64, 256, None, None) == INVALID   # q overlaps x
    g = lib.ffn_gateup_acc_tiled               # h, h_absmax, x, xs, w, ws, N, C, H
    assert g(A, M, A, None, A, S, 64, 256, 768, None) == INVALID           # no x_scale
    assert g(A, M, A, M, A, S, 64, 256, 768, None) == INVALID              # abs-max aliases x_scale
    assert g(A, M, A, Z, A, S, 64, 200, 768, None) == UNSUPPORTED          # C % 128
    assert g(A, M, A, Z, A, S, 64, 256, 100, None) == UNSUPPORTED          # H % 128
    assert g(A, M, A, Z, A, S, (1 << 20), 4096, 768, None) == UNSUPPORTED  # > 4 GiB operand
    assert g(A, M, MIS, Z, A, S, 64, 256, 768, None) == UNSUPPORTED
    k = lib.ffn_gateup_swiglu_quant_tiled      # q, q_scale, h_absmax, known, x, xs, w, ws, N, C, H
    assert k(A, S, M, None, A, Z, A, 0x50000, 64, 256, 768, None) == INVALID   # no known abs-max
    assert k(A, S, M, M, A, Z, A, 0x50000, 64, 256, 768, None) == INVALID      # known aliases h_absmax
    assert k(A, S, M, 0x60000, A, S, A, 0x50000, 64, 256, 768, None) == INVALID  # q_scale aliases x_scale
    assert k(A, S, M, 0x60000, A, Z, A, 0x50000, 64, 256, 100, None) == UNSUPPORTED
    d = lib.ffn_down_tiled                     # out, h, hs, w, ws, N, H, C
    assert d(A, A, None, A, S, 64, 768, 256, None) == INVALID
    assert d(A, A, Z, A, S, 64, 700, 256, None) == UNSUPPORTED
    assert d(A, A, Z, A, S, 64, 768, 200, None) == UNSUPPORTED
    assert d(None, A, Z, A, S, 64, 768, 256, None) == INVALID
    r = lib.ffn_rmsnorm_fwd_tiled              # y, rstd, res, absmax, inp, addend, w, eps, N, C
    Y, X = 0x100000, 0x200000
    assert r(Y, A, None, None, X, None, A, 1e-5, 64, 200, None) == UNSUPPORTED  # C % 32
    assert r(X + 64, A, None, None, X, None, A, 1e-5, 64, 256, None) == INVALID  # tiled y overlaps inp
    assert "overlap" in _err(lib)
    assert r(0x300040, A, 0x400000, None, X, 0x300000, A, 1e-5, 64, 256, None) == INVALID  # overlaps addend
    gb = lib.ffn_gateup_tiled_bf16             # h, absmax, x, w, N, C, H
    assert gb(A, None, A, A, 64, 200, 768, None) == UNSUPPORTED
    assert gb(A, None, A, A, 64, 256, 100, None) == UNSUPPORTED
    assert gb(None, None, A, A, 64, 256, 768, None) == INVALID
    assert gb(A, None, MIS, A, 64, 256, 768, None) == UNSUPPORTED
    TILED = 4
    tn = lib.ffn_matmul_tn                     # out, a, as, b, bs, dtype, flags, M, N, K
    assert tn(A, 0x20000, S, 0x30000, Z, 0, TILED, 64, 256, 256, None) == UNSUPPORTED   # bf16 operands
    assert tn(A, 0x20000, S, 0x30000, Z, 1, 8, 64, 256, 256, None) == INVALID          # unknown flag
    sb = lib.ffn_matmul_tn_swiglu_bwd          # dgu, absmax, a, as, b, bs, gu, dtype, flags, M, H, K
    assert sb(A, None, 0x20000, S, 0x30000, Z, 0x40000, 0, TILED, 64, 256, 256, None) == UNSUPPORTED
    tt = lib.ffn_transpose_tiled               # out, in, rows, cols, ld_out
    assert tt(A, 0x20000, 64, 96, 128, None) == UNSUPPORTED     # cols % 64
    assert tt(A, 0x20000, 64, 128, 80, None) == UNSUPPORTED     # ld_out % 64
    assert tt(A, 0x20000, 128, 128, 64, None) == INVALID        # ld_out < rows
    assert tt(A, A, 64, 128, 128, None) == INVALID              # out aliases in
    qt = lib.ffn_quant_transpose_tiled         # q_t, q, scale, x, absmax, clear, dtype, rows, cols, ld_out
    assert qt(A, None, S, 0x20000, M, None, 1, 64, 96, 128, None) == UNSUPPORTED
    assert qt(A, None, S, 0x20000, S, None, 1, 64, 128, 128, None) == INVALID   # scale aliases absmax
    assert qt(A, None, S, 0x20000, M, M, 1, 64, 128, 128, None) == INVALID      # clear aliases absmax
    assert qt(A, None, S, 0x20000, M, None, 0, 64, 128, 128, None) == INVALID   # bf16 codes
    db = lib.ffn_down_tiled_bf16               # out, h, w, N, H, C
    assert db(A, A, A, 64, 700, 256, None) == UNSUPPORTED
    assert db(A, None, A, 64, 768, 256, None) == INVALID
    assert db(A, A, A, -1, 768, 256, None) == INVALID


def test_decode_validation(lib):
    f = lib.ffn_decode_gemv
    args = [A, A + 4096, A + 8192, A, A, A, A, A, A]
    assert f(*args, 33, 4096, 14336, None) == UNSUPPORTED
    assert f(*args, 1, 4000, 14336, None) == UNSUPPORTED
    assert f(*args, -1, 4096, 14336, None) == INVALID
    bad = list(args)
    bad[4] = None
    assert f(*bad, 1, 4096, 14336, None) == INVALID
    alias = list(args)
    alias[1] = alias[2]
    assert f(*alias, 1, 4096, 14336, None) == INVALID
    mis = list(args)
    mis[3] = MIS
    assert f(*mis, 1, 4096, 14336, None) == UNSUPPORTED


def test_decode_packed_validation(lib):
    B, C_, D, E = 0x20000, 0x30000, 0x40000, 0x50000
    p = lib.ffn_decode_pack_weight   # packed, w, rows, cols
    assert p(A, B, 24, 256, None) == UNSUPPORTED        # rows % 16
    assert p(A, B, 32, 200, None) == UNSUPPORTED        # cols % 128
    assert p(A, A, 32, 256, None) == INVALID            # in place
    assert p(None, B, 32, 256, None) == INVALID
    assert p(A, MIS, 32, 256, None) == UNSUPPORTED
    ws = lib.ffn_decode_packed_workspace_bytes

    def slices(C, H):   # the header's rule for the down pass's K slices
        n = H // 64
        return max(1, min(n, max(256 // (C // 128), -(-n // 64))))

    def one_block(C, H):   # x and h in fragment order + fp32 partial sums
        return 32 * (C + H) + 64 * slices(C, H) * C

    assert slices(3584, 18944) == 9 and slices(4096, 14336) == 8 and slices(128, 128) == 2
    assert ws(16, 3584, 18944) == one_block(3584, 18944) and ws(1, 256, 256) == one_block(256, 256)
    assert ws(17, 3584, 18944) == max(64 * (3584 + 18944), one_block(3584, 18944))
    assert ws(32, 8192, 256) == max(64 * (8192 + 256), one_block(8192, 256))
    assert all(ws(m, 1152, 4096) <= ws(m + 1, 1152, 4096) for m in range(32))   # never smaller for more tokens
    assert ws(33, 256, 256) == -1 and ws(-1, 256, 256) == -1
    g = lib.ffn_decode_gemv_packed   # out, h, ws, x, wg, sg, wu, su, wd, sd, M, C, H
    assert g(A, B, None, D, A, A, A, A, A, A, 16, 256, 768, None) == INVALID       # no workspace
    assert g(A, B, B, D, A, A, A, A, A, A, 16, 256, 768, None) == INVALID          # workspace aliases h
    assert g(A, B, E, D, A, A, A, A, A, A, 33, 256, 768, None) == UNSUPPORTED      # M > 32
    assert g(A, B, E, D, A, A, A, A, A, A, 16, 200, 768, None) == UNSUPPORTED      # C % 128
    assert g(A, B, MIS, D, A, A, A, A, A, A, 16, 256, 768, None) == UNSUPPORTED    # misaligned workspace
    assert g(A, B, E, D, A, None, A, A, A, A, 16, 256, 768, None) == INVALID       # no gate scales
    n = lib.ffn_decode_gemv_packed_noalloc   # out, h, x, wg, sg, wu, su, wd, sd, M, C, H
    assert lib.ffn_decode_noalloc_scratch_bytes() == 8 << 20
    assert n(A, B, D, A, A, A, A, A, A, 16, 131072, 128, None) == UNSUPPORTED      # workspace beyond the scratch
    assert "scratch" in _err(lib)
    assert n(A, B, D, A, None, A, A, A, A, 16, 256, 768, None) == INVALID          # no gate scales
    assert n(A, B, D, A, A, A, A, A, A, 33, 256, 768, None) == UNSUPPORTED         # M > 32


def test_decode_arm_and_bf16_validation(lib):
    B, C_, D = 0x20000, 0x30000, 0x40000
    f = lib.ffn_decode_gemv_arm   # out, h, gu, x, wg, sg, wu, su, wd, sd, arm, M, C, H
    assert f(A, B, C_, D, A, A, A, A, A, A, 7, 1, 256, 768, None) == INVALID          # unknown arm
    assert f(A, B, None, D, A, A, A, A, A, A, 1, 1, 256, 768, None) == INVALID        # SiLU-input arm needs gu
    assert f(A, B, B, D, A, A, A, A, A, A, 2, 1, 256, 768, None) == INVALID           # gu aliases h
    assert f(A, B, C_, D, A, A, A, A, A, A, 1, 5, 256, 768, None) == UNSUPPORTED      # M > 4 off the split arm
    assert f(A, B, None, D, A, A, A, A, A, A, 0, 33, 256, 768, None) == UNSUPPORTED   # M > 32
    assert f(A, B, C_, D, A, None, A, A, A, A, 0, 1, 256, 768, None) == INVALID       # no gate scales
    assert f(A, B, MIS, D, A, A, A, A, A, A, 1, 1, 256, 768, None) == UNSUPPORTED     # misaligned gu
    g = lib.ffn_decode_gemv_bf16  # out, h, x, wg, wu, wd, M, C, H
    assert g(A, B, D, A, A, None, 1, 256, 768, None) == INVALID                       # no down weight
    assert g(A, B, D, A, A, A, 5, 256, 768, None) == UNSUPPORTED                      # M > 4
    assert g(A, B, D, A, A, A, 1, 200, 768, None) == UNSUPPORTED                      # C % 128
    assert g(A, A, D, A, A, A, 1, 256, 768, None) == INVALID                          # h aliases out
    assert g(A, B, D, A, A, A, 1, 32768, 32768, None) == UNSUPPORTED                  # > 2 GiB of weights


def test_backward_validation(lib):
    B_, C_, D = 0x20000, 0x30000, 0x40000
    m = lib.ffn_matmul_tn  # out, a, sa, b, sb, dtype, flags, M, N, K
    assert m(None, B_, None, C_, None, 0, 0, 64, 256, 128, None) == INVALID
    assert m(A, B_, None, C_, None, 1, 0, 64, 256, 128, None) == INVALID           # E4M3 without scales
    assert m(A, B_, None, C_, None, 2, 0, 64, 256, 128, None) == INVALID           # E5M2 without scales
    assert m(A, B_, None, C_, None, 5, 0, 64, 256, 128, None) == INVALID           # unknown dtype
    assert m(A, B_, None, C_, None, 0, 8, 64, 256, 128, None) == INVALID           # unknown flag bit
    assert m(A, B_, D, C_, D, 2, 0, 64, 200, 128, None) == UNSUPPORTED             # E5M2, N % 128
    assert m(A, B_, None, C_, None, 0, 0, 64, 200, 128, None) == UNSUPPORTED       # N % 128
    assert m(A, B_, None, C_, None, 0, 0, 64, 256, 96, None) == UNSUPPORTED        # K % 128
    assert m(A, A, None, C_, None, 0, 0, 64, 256, 128, None) == INVALID            # out aliases a
    assert m(A, B_, None, MIS, None, 0, 0, 64, 256, 128, None) == UNSUPPORTED      # misaligned b
    assert m(A, B_, None, C_, None, 0, 0, -1, 256, 128, None) == INVALID
    f = lib.ffn_matmul_tn_swiglu_bwd  # dgu, absmax, a, sa, b, sb, gu, dtype, flags, M, H, K
    assert f(A, None, B_, None, C_, None, None, 0, 0, 64, 256, 128, None) == INVALID      # no gu
    assert f(A, None, B_, None, C_, None, D, 1, 0, 64, 256, 128, None) == INVALID         # FP8 without scales
    assert f(A, None, B_, None, C_, None, D, 7, 0, 64, 256, 128, None) == INVALID         # unknown dtype
    assert f(A, None, B_, None, C_, None, D, 0, 1, 64, 256, 128, None) == INVALID         # accumulate: no
    assert f(A, None, B_, None, C_, None, D, 0, 0, 64, 200, 128, None) == UNSUPPORTED     # H % 128
    assert f(A, None, B_, None, C_, None, D, 0, 2, 64, 256, 96, None) == UNSUPPORTED      # K % 128
    assert f(B_, None, B_, None, C_, None, D, 0, 0, 64, 256, 128, None) == INVALID        # dgu aliases a
    assert f(A, None, B_, None, C_, None, MIS, 0, 0, 64, 256, 128, None) == UNSUPPORTED   # misaligned gu
    assert f(A, None, B_, None, C_, None, D, 0, 0, -1, 256, 128, None) == INVALID
    assert f(A, 0x80000, B_, 0x80000, C_, 0x90000, D, 1, 0, 64, 256, 128, None) == INVALID  # absmax aliases a_scale
    assert f(A, 0x90000, B_, 0x80000, C_, 0x90000, D, 1, 0, 64, 256, 128, None) == INVALID  # absmax aliases b_scale
    t = lib.ffn_transpose  # out, in, rows, cols, ld_out, elt
    assert t(A, B_, 37, 64, 48, 3, None) == INVALID                                # element size
    assert t(A, B_, 37, 64, 32, 2, None) == INVALID                                # ld_out < rows
    assert t(A, B_, 37, 40, 48, 2, None) == UNSUPPORTED                            # cols % 16
    assert t(A, B_, 37, 64, 40, 2, None) == UNSUPPORTED                            # ld_out % 16
    assert t(A, A, 37, 64, 48, 2, None) == INVALID                                 # in place
    assert t(A, MIS, 37, 64, 48, 1, None) == UNSUPPORTED
    q = lib.ffn_quant_transpose  # q_t, q, scale, x, absmax, code dtype, rows, cols, ld_out
    assert q(A, None, B_, C_, None, 1, 37, 64, 48, None) == INVALID                # no abs-max
    assert q(A, None, B_, C_, D, 1, 37, 64, 32, None) == INVALID                   # ld_out < rows
    assert q(A, A, B_, C_, D, 2, 37, 64, 48, None) == INVALID                      # q aliases q_t
    assert q(A, MIS, B_, C_, D, 1, 37, 64, 48, None) == UNSUPPORTED                # misaligned q
    assert q(A, None, B_, C_, D, 0, 37, 64, 48, None) == INVALID                   # bf16 is no code format
    assert q(A, None, B_, C_, D, 3, 37, 64, 48, None) == INVALID                   # unknown code format
    assert q(A, None, D, C_, D, 1, 37, 64, 48, None) == INVALID                    # scale aliases absmax
    assert "scale and absmax alias" in _err(lib)
    g = lib.ffn_swiglu_bwd  # dgu, absmax, dh, gu, N, H
    assert g(A, None, A, C_, 4, 64, None) == INVALID                               # dgu aliases dh
    assert g(A, None, B_, C_, 4, 60, None) == UNSUPPORTED                          # H % 8
    assert g(A, None, B_, None, 4, 64, None) == INVALID
    r = lib.ffn_rmsnorm_bwd  # dinp, dweight, scratch, dres, dy, r, w, rstd, absmax, N, C
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, None, 4, 8200, None) == UNSUPPORTED  # C > 8192
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, None, 4, 100, None) == UNSUPPORTED   # C % 8
    assert r(A, B_, None, A, D, 0x50000, 0x60000, 0x70000, None, 4, 256, None) == INVALID     # no scratch
    assert r(A, B_, C_, A, A, 0x50000, 0x60000, 0x70000, None, 4, 256, None) == INVALID       # dinp aliases dy
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, None, -4, 256, None) == INVALID
    sb = lib.ffn_rmsnorm_bwd_scratch_bytes
    assert sb(0, 4096) == 0 and sb(8192, 4096) == 512 * 4096 * 4 and sb(3, 256) == 3 * 256 * 4
    assert sb(4, 9000) == -1


def test_backward_absmax_accumulating_forms_validation(lib):
    B_, C_, D, W1, W2 = 0x20000, 0x30000, 0x40000, 0x80000, 0x90000
    f = lib.ffn_matmul_tn_swiglu_bwd_acc  # dgu, absmax, a, sa, b, sb, gu, dtype, flags, M, H, K
    assert f(A, None, B_, None, C_, None, D, 0, 0, 64, 256, 128, None) == INVALID          # absmax required
    assert "absmax is NULL" in _err(lib)
    assert f(A, W1, B_, None, C_, None, D, 1, 0, 64, 256, 128, None) == INVALID            # FP8 without scales
    assert f(A, W1, B_, W1, C_, W2, D, 1, 0, 64, 256, 128, None) == INVALID                # absmax aliases a_scale
    assert f(A, W1, B_, None, C_, None, D, 0, 0, 64, 200, 128, None) == UNSUPPORTED        # H % 128
    assert "ffn_matmul_tn_swiglu_bwd_acc" in _err(lib)
    q = lib.ffn_quant_transpose_clear  # q_t, q, scale, x, absmax, clear, code dtype, rows, cols, ld_out
    assert q(A, None, B_, C_, D, None, 1, 37, 64, 48, None) == INVALID                     # clear required
    assert q(A, None, B_, C_, D, D, 1, 37, 64, 48, None) == INVALID                        # clear aliases absmax
    assert "clear must not alias" in _err(lib)
    assert q(A, None, B_, C_, D, B_, 1, 37, 64, 48, None) == INVALID                       # clear aliases scale
    assert q(A, None, D, C_, D, W1, 1, 37, 64, 48, None) == INVALID                        # scale aliases absmax
    assert q(A, None, B_, C_, D, W1, 0, 37, 64, 48, None) == INVALID                       # bf16 is no code format
    assert q(A, None, B_, C_, D, W1, 1, 37, 64, 32, None) == INVALID                       # ld_out < rows
    g = lib.ffn_swiglu_bwd_acc  # dgu, absmax, dh, gu, N, H
    assert g(A, None, B_, C_, 4, 64, None) == INVALID                                      # absmax required
    assert g(A, W1, A, C_, 4, 64, None) == INVALID                                         # dgu aliases dh
    assert g(A, W1, B_, C_, 4, 60, None) == UNSUPPORTED                                    # H % 8
    r = lib.ffn_rmsnorm_bwd_acc  # dinp, dweight, scratch, dres, dy, r, w, rstd, absmax, clear, N, C
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, None, None, 4, 256, None) == INVALID  # absmax required
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, W1, W1, 4, 256, None) == INVALID      # clear aliases absmax
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, W1, W2, 4, 8200, None) == UNSUPPORTED  # C > 8192
    assert r(A, B_, C_, A, A, 0x50000, 0x60000, 0x70000, W1, W2, 4, 256, None) == INVALID      # dinp aliases dy
    assert r(A, B_, C_, A, D, 0x50000, 0x60000, 0x70000, W1, None, -4, 256, None) == INVALID


def test_binding_rejects_host_tensors_and_short_buffers():
    if not os.path.exists(LIB):
        pytest.skip("libffn.so not built")
    import torch
    import transformer_ffn_block_residual_amd as F
    with pytest.raises(F.FFNError):
        F.ffn_swiglu(torch.empty(8, dtype=torch.bfloat16), None, torch.empty(16, dtype=torch.bfloat16), 1, 8)
