"""The tiled operand layout of the e4m3 prefill GEMMs.

The tiled entry points run the same kernels as the row-major ones with only
the global load (and, for the codes of h, store) offsets changed, so their
results must equal the row-major results bit for bit; the row-major results
are themselves checked against the oracle elsewhere.  The layout is checked
against a numpy re-indexing written from the header's definition, which a
CPU test pins to a per-element loop over that definition.
"""

import numpy as np
import pytest
import torch

from transformer_ffn_block_residual_amd import workloads as W
from tests.gpu_util import say, dev_bf16, dev_u8, dev_f32, host_bits, host_u8, empty_bf16, empty_f32, empty_u8


def tiled_ref(a):
    """The tiled layout of a [rows, rb] uint8 array (rb % 64 == 0), whole
    64-row groups, pad rows zero: block (g, s, i) at g*64*rb + s*4096 + i*1024
    holds, at 16*l + b, byte 64 s + 16 ((l % 4) ^ (l // 16)) + b of row
    64 g + 16 i + l // 4."""
    rows, rb = a.shape
    G, S = -(-rows // 64), rb // 64
    p = np.zeros((G * 64, rb), np.uint8)
    p[:rows] = a
    v = p.reshape(G, 4, 16, S, 4, 16)                  # [g, i, row in sub-group, s, chunk, b]
    lane = np.arange(64)
    lr, ch = lane // 4, (lane % 4) ^ (lane // 16)
    t = v[:, :, lr, :, ch, :]                          # [lane, g, i, s, b]
    return np.ascontiguousarray(t.transpose(1, 3, 2, 0, 4)).reshape(-1)


def tiled_ref_loop(a):
    """The same layout, one byte at a time from the definition."""
    rows, rb = a.shape
    G = -(-rows // 64)
    out = np.zeros(G * 64 * rb, np.uint8)
    for r in range(rows):
        g, i, lr = r // 64, (r % 64) // 16, r % 16
        for c in range(rb):
            s, chunk, b = c // 64, (c % 64) // 16, c % 16
            lane = 4 * lr + (chunk ^ (lr // 4))
            out[g * 64 * rb + s * 4096 + i * 1024 + 16 * lane + b] = a[r, c]
    return out


@pytest.mark.parametrize("rows,rb", [(64, 64), (16, 128), (100, 192), (130, 256)])
def test_tiled_reference_matches_its_definition(rows, rb):
    a = np.random.default_rng(rows * rb).integers(0, 256, (rows, rb)).astype(np.uint8)
    assert np.array_equal(tiled_ref(a), tiled_ref_loop(a))


def _codes(shape, seed, top=0x58):
    """Random finite e4m3 codes with magnitudes up to about 2^4, both signs."""
    rng = np.random.default_rng(seed)
    mag = rng.integers(0, top, shape)
    return (mag | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_ffn_block_residual_amd import binding
    return binding


def _pack(B, q, rows, rb):
    t = empty_u8(B.ffn_tile_bytes(rows, rb)).fill_(0xA5)
    B.ffn_tile_pack(t, q, rows, rb)
    return t


@pytest.mark.gpu
@pytest.mark.parametrize("rows,rb", [(64, 64), (1, 128), (100, 192), (300, 3584), (37888, 3584)])
def test_tile_pack_layout(B, rows, rb):
    say(f"tile pack rows={rows} row_bytes={rb}")
    a = np.random.default_rng(rows + rb).integers(0, 256, (rows, rb)).astype(np.uint8)
    t = _pack(B, dev_u8(a), rows, rb)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(t), tiled_ref(a))   # pad rows written as zeros


@pytest.mark.gpu
@pytest.mark.parametrize("rows,cols", [(1, 128), (64, 256), (300, 384), (8192, 3584)])
def test_quant_tiled_is_the_row_major_codes_moved(B, rows, cols):
    say(f"quant tiled rows={rows} cols={cols}")
    x = W.normal_bf16((rows, cols), 1.0, rows + cols, 11)
    xd = dev_bf16(x)
    am = dev_f32(np.array([3.5], np.float32))          # values past it saturate
    q, s = empty_u8(rows, cols), empty_f32(1)
    clear1 = dev_f32(np.array([7.0], np.float32))
    B.ffn_quant_absmax_clear(q, s, am, xd, rows * cols, clear1)
    qt, st = empty_u8(B.ffn_tile_bytes(rows, cols)).fill_(0xA5), empty_f32(1)
    clear2 = dev_f32(np.array([7.0], np.float32))
    B.ffn_quant_absmax_clear_tiled(qt, st, am, xd, rows, cols, clear2)
    torch.cuda.synchronize()
    want = tiled_ref(host_u8(q).reshape(rows, cols))
    got = host_u8(qt)
    valid = tiled_ref(np.ones((rows, cols), np.uint8)).astype(bool)
    assert np.array_equal(got[valid], want[valid])
    assert np.all(got[~valid] == 0xA5)                  # rows past `rows` are left as found
    assert torch.equal(st, s) and clear2.item() == 0.0


# (N, C, H): ragged token counts (a partial 64-row group and empty slabs in
# the last tile), output widths that are not a multiple of 256 (down), a
# persistent grid of several rounds, and the Qwen2-7B-shaped prefill.
GEMM_SHAPES = [(1, 128, 128), (64, 256, 128), (300, 512, 384), (1000, 384, 640), (4096, 1024, 4096),
               (8192, 3584, 18944)]


@pytest.mark.gpu
@pytest.mark.parametrize("N,C,H", GEMM_SHAPES)
def test_tiled_gemms_equal_the_row_major_ones(B, N, C, H):
    say(f"tiled gemms N={N} C={C} H={H}")
    x, wgu = dev_u8(_codes((N, C), N + 1)), dev_u8(_codes((2 * H, C), C + 2))
    hq, wd = dev_u8(_codes((N, H), N + 3)), dev_u8(_codes((C, H), H + 4))
    sx, sw = dev_f32(np.array([0.011], np.float32)), dev_f32(np.array([0.013], np.float32))
    xt, wgut, hqt, wdt = _pack(B, x, N, C), _pack(B, wgu, 2 * H, C), _pack(B, hq, N, H), _pack(B, wd, C, H)
    # gate+up with SwiGLU, accumulating abs-max
    h1, h2 = empty_bf16(N, H), empty_bf16(N, H)
    am1, am2 = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    B.ffn_gateup_acc(h1, am1, x, sx, wgu, sw, B.FFN_E4M3, N, C, H)
    B.ffn_gateup_acc_tiled(h2, am2, xt, sx, wgut, sw, N, C, H)
    # down
    o1, o2 = empty_bf16(N, C), empty_bf16(N, C)
    B.ffn_down(o1, hq, sx, wd, sw, B.FFN_E4M3, N, H, C)
    B.ffn_down_tiled(o2, hqt, sx, wdt, sw, N, H, C)
    # gate+up with the codes of h under a known abs-max
    known = dev_f32(np.array([0.75], np.float32))
    q1, qs1, qa1 = empty_u8(N, H), empty_f32(1), empty_f32(1)
    q2, qs2, qa2 = empty_u8(B.ffn_tile_bytes(N, H)).fill_(0xA5), empty_f32(1), empty_f32(1)
    B.ffn_gateup_swiglu_quant(q1, qs1, qa1, known, x, sx, wgu, sw, B.FFN_E4M3, N, C, H)
    B.ffn_gateup_swiglu_quant_tiled(q2, qs2, qa2, known, xt, sx, wgut, sw, N, C, H)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(am1, am2)
    assert torch.equal(o1, o2)
    want = tiled_ref(host_u8(q1).reshape(N, H))
    got = host_u8(q2)
    valid = tiled_ref(np.ones((N, H), np.uint8)).astype(bool)
    assert np.array_equal(got[valid], want[valid])
    assert np.all(got[~valid] == 0xA5)                  # rows past N are not written
    assert torch.equal(qs1, qs2) and torch.equal(qa1, qa2)


@pytest.mark.gpu
def test_tiled_token_rows_past_n_do_not_matter(B):
    """The rows past N of the last 64-row group are don't-care: filling them
    with other codes (NaN codes included) changes nothing that is stored."""
    N, C, H = 100, 256, 256
    say("tiled pad rows")
    x, wgu = _codes((N, C), 5), dev_u8(_codes((2 * H, C), 6))
    wgut = _pack(B, wgu, 2 * H, C)
    sx, sw = dev_f32(np.array([0.02], np.float32)), dev_f32(np.array([0.02], np.float32))
    res = []
    for fill in (0, 0x7F):
        pad = np.full((128, C), fill, np.uint8)
        pad[:N] = x
        xt = empty_u8(B.ffn_tile_bytes(N, C))
        B.ffn_tile_pack(xt, dev_u8(pad), 128, C)          # 128 rows: two whole groups
        h, am = empty_bf16(N, H), torch.zeros(1, device="cuda")
        B.ffn_gateup_acc_tiled(h, am, xt, sx, wgut, sw, N, C, H)
        res.append((h, am))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.fixture(scope="module")
def blk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from transformer_ffn_block_residual_amd import block
    return block


@pytest.mark.gpu
@pytest.mark.parametrize("N,C,H", [(300, 512, 384), (8192, 3584, 18944)])
def test_tiled_block_equals_the_row_major_block(blk, B, N, C, H):
    """PrefillBlock(tiled=True): both forwards give the row-major block's
    outputs bit for bit (and its codes, moved)."""
    say(f"tiled block N={N} C={C} H={H}")
    d = W.block_inputs(N, C, H, seed=N + 5, outliers=True)
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    res = {}
    for tiled in (False, True):
        b = blk.PrefillBlock(N, C, H, 1e-5, True, tiled=tiled)
        b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
        out = b.forward_zero_once(inp, add).clone()
        st = {n: getattr(b, n).clone() for n in ("r", "y", "rstd", "h", "am_h", "am_y", "s_y", "s_h", "qy", "qh")}
        known, am_out = dev_f32(np.array([0.9], np.float32)), empty_f32(1)
        out_k = b.forward_known_h_absmax(inp, add, known, am_out).clone()
        res[tiled] = (out, st, out_k, am_out.clone(), b.qh.clone(), b.s_h.clone())
    torch.cuda.synchronize()
    (o0, s0, k0, a0, qh0, sh0), (o1, s1, k1, a1, qh1, sh1) = res[False], res[True]
    assert torch.equal(o0, o1) and torch.equal(k0, k1) and torch.equal(a0, a1) and torch.equal(sh0, sh1)
    for n in ("r", "y", "rstd", "h", "am_h", "am_y", "s_y", "s_h"):
        assert torch.equal(s0[n], s1[n]), n
    for n, rb in (("qy", C), ("qh", H)):
        valid = tiled_ref(np.ones((N, rb), np.uint8)).astype(bool)
        assert np.array_equal(host_u8(s1[n])[valid], tiled_ref(host_u8(s0[n]).reshape(N, rb))[valid]), n
    valid = tiled_ref(np.ones((N, H), np.uint8)).astype(bool)
    assert np.array_equal(host_u8(qh1)[valid], tiled_ref(host_u8(qh0).reshape(N, H))[valid])


@pytest.mark.gpu
def test_tiled_block_replays_from_a_hip_graph(blk, B):
    N, C, H = 300, 512, 384
    say("tiled block graph replay")
    d = W.block_inputs(N, C, H, seed=79)
    b = blk.PrefillBlock(N, C, H, 1e-5, True, tiled=True)
    b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    b.forward_zero_once(inp, add)
    torch.cuda.synchronize()
    names = ["r", "y", "rstd", "am_y", "h", "am_h", "out", "qy", "s_y", "qh", "s_h"]
    eager = {n: getattr(b, n).clone() for n in names}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        b.forward_zero_once(inp, add)
    scratch_y, scratch_rstd = empty_bf16(N, C), empty_f32(N)
    masks = {n: torch.from_numpy(tiled_ref(np.ones((N, rb), np.uint8)).astype(bool)).cuda()
             for n, rb in (("qy", C), ("qh", H))}
    for rep in range(3):
        for n in names:
            if n not in ("am_y", "am_h"):      # the zero-once words must stay as the last call left them
                getattr(b, n).zero_()
        B.ffn_rmsnorm_fwd(scratch_y, scratch_rstd, None, None, inp, None, b.w_norm, 1e-5, N, C)  # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            if n in masks:      # the rows past N of the tiled codes are don't-care
                assert torch.equal(getattr(b, n)[masks[n]], eager[n][masks[n]]), (rep, n)
            else:
                assert torch.equal(getattr(b, n), eager[n]), (rep, n)


@pytest.mark.gpu
def test_tiled_zero_rows(B):
    """No rows: nothing is written but the per-tensor words, as for the
    row-major calls (the _acc word as found, the known abs-max's scale, an
    abs-max of no elements 0, the cleared word 0)."""
    say("tiled zero rows")
    C, H = 256, 256
    xs, ws = dev_f32([0.5]), dev_f32([0.25])
    x, w, wd = empty_u8(64 * C).zero_(), empty_u8(2 * H * C).zero_(), empty_u8(C * H).zero_()
    h = empty_bf16(1, H).fill_(3.0)
    acc = dev_f32([7.0])
    B.ffn_gateup_acc_tiled(h, acc, x, xs, w, ws, 0, C, H)
    q, qs, ham = empty_u8(64 * H).fill_(0x11), dev_f32([-1.0]), dev_f32([7.0])
    B.ffn_gateup_swiglu_quant_tiled(q, qs, ham, dev_f32([3.5]), x, xs, w, ws, 0, C, H)
    out = empty_bf16(1, C).fill_(2.0)
    B.ffn_down_tiled(out, empty_u8(64 * H).zero_(), xs, wd, ws, 0, H, C)
    qy, sy, clear = empty_u8(64 * C).fill_(0x22), dev_f32([-1.0]), dev_f32([5.0])
    B.ffn_quant_absmax_clear_tiled(qy, sy, dev_f32([3.5]), empty_bf16(1, C).zero_(), 0, C, clear)
    packed = empty_u8(64 * C).fill_(0x33)
    B.ffn_tile_pack(packed, empty_u8(C).zero_(), 0, C)
    torch.cuda.synchronize()
    assert acc.item() == 7.0 and ham.item() == 0.0 and clear.item() == 0.0
    assert qs.item() == sy.item() == np.float32(3.5) / np.float32(448.0)
    assert torch.all(h == 3.0) and torch.all(out == 2.0)
    assert torch.all(q == 0x11) and torch.all(qy == 0x22) and torch.all(packed == 0x33)


# ----------------------------------------------------------------------------- the bf16 block on tiled operands

def _bytes_of_bf16(t, rows, cols):
    """A row-major bf16 device tensor as its [rows, 2 cols] bytes."""
    return host_bits(t).reshape(rows, cols).view(np.uint8).reshape(rows, 2 * cols)


@pytest.mark.gpu
@pytest.mark.parametrize("N,C,add", [(1, 128, False), (100, 512, True), (300, 4096, True), (64, 8192, False),
                                     (8192, 3584, True)])
def test_rmsnorm_tiled_y_is_the_row_major_y_moved(B, N, C, add):
    say(f"rmsnorm tiled y N={N} C={C} add={add}")
    d = W.block_inputs(N, C, 128, seed=N + C)
    inp, w = dev_bf16(d["inp"]), dev_bf16(d["w_norm"])
    addend = dev_bf16(d["addend"]) if add else None
    y1, r1, s1, a1 = empty_bf16(N, C), empty_bf16(N, C) if add else None, empty_f32(N), empty_f32(1)
    B.ffn_rmsnorm_fwd(y1, s1, r1, a1, inp, addend, w, 1e-5, N, C)
    y2 = empty_bf16(B.ffn_tile_bytes(N, 2 * C) // 2).fill_(-5.0)
    r2, s2, a2 = empty_bf16(N, C) if add else None, empty_f32(N), empty_f32(1)
    B.ffn_rmsnorm_fwd_tiled(y2, s2, r2, a2, inp, addend, w, 1e-5, N, C)
    torch.cuda.synchronize()
    valid = tiled_ref(np.ones((N, 2 * C), np.uint8)).astype(bool)
    got = host_bits(y2).view(np.uint8)
    assert np.array_equal(got[valid], tiled_ref(_bytes_of_bf16(y1, N, C))[valid])
    pad = host_bits(y2).view(np.uint8)[~valid]
    assert np.array_equal(pad, np.tile(host_bits(empty_bf16(1).fill_(-5.0)).view(np.uint8), pad.size // 2))
    assert torch.equal(s1, s2) and torch.equal(a1, a2) and (not add or torch.equal(r1, r2))


@pytest.mark.gpu
@pytest.mark.parametrize("N,C,H", [(1, 128, 128), (300, 512, 384), (1000, 384, 640), (4096, 4096, 14336)])
def test_tiled_bf16_gemms_equal_the_row_major_ones(B, N, C, H):
    say(f"tiled bf16 gemms N={N} C={C} H={H}")
    x = W.normal_bf16((N, C), 1.0, N + 1, 21)
    wgu = W.normal_bf16((2 * H, C), 0.05, C + 2, 22)
    hh = W.normal_bf16((N, H), 1.0, N + 3, 23)
    wd = W.normal_bf16((C, H), 0.05, H + 4, 24)
    xd, wgud, hd, wdd = dev_bf16(x), dev_bf16(wgu), dev_bf16(hh), dev_bf16(wd)

    def tiled(t, rows, cols):
        o = empty_bf16(B.ffn_tile_bytes(rows, 2 * cols) // 2)
        B.ffn_tile_pack(o.view(torch.uint8), t.view(torch.uint8), rows, 2 * cols)
        return o
    xt, wgut, ht, wdt = tiled(xd, N, C), tiled(wgud, 2 * H, C), tiled(hd, N, H), tiled(wdd, C, H)
    h1, am1 = empty_bf16(N, H), empty_f32(1)
    B.ffn_gateup(h1, am1, xd, None, wgud, None, B.FFN_BF16, 1, N, C, H)
    h2, am2 = empty_bf16(B.ffn_tile_bytes(N, 2 * H) // 2).fill_(-5.0), empty_f32(1)
    B.ffn_gateup_tiled_bf16(h2, am2, xt, wgut, N, C, H)
    o1, o2 = empty_bf16(N, C), empty_bf16(N, C)
    B.ffn_down(o1, hd, None, wdd, None, B.FFN_BF16, N, H, C)
    B.ffn_down_tiled_bf16(o2, ht, wdt, N, H, C)
    torch.cuda.synchronize()
    valid = tiled_ref(np.ones((N, 2 * H), np.uint8)).astype(bool)
    got = host_bits(h2).view(np.uint8)
    assert np.array_equal(got[valid], tiled_ref(_bytes_of_bf16(h1, N, H))[valid])
    assert torch.equal(am1, am2) and torch.equal(o1, o2)


@pytest.mark.gpu
@pytest.mark.parametrize("N,C,H", [(300, 512, 384), (4096, 4096, 14336)])
def test_tiled_bf16_block_equals_the_row_major_block(blk, B, N, C, H):
    say(f"tiled bf16 block N={N} C={C} H={H}")
    d = W.block_inputs(N, C, H, seed=N + 7)
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    res = {}
    for tiled in (False, True):
        b = blk.PrefillBlock(N, C, H, 1e-5, False, tiled=tiled)
        b.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
        out = b.forward_zero_once(inp, add).clone()
        res[tiled] = (out, b.r.clone(), b.rstd.clone(), b.y.clone(), b.h.clone())
    torch.cuda.synchronize()
    (o0, r0, s0, y0, h0), (o1, r1, s1, y1, h1) = res[False], res[True]
    assert torch.equal(o0, o1) and torch.equal(r0, r1) and torch.equal(s0, s1)
    for a, b_, cols in ((y0, y1, C), (h0, h1, H)):
        valid = tiled_ref(np.ones((N, 2 * cols), np.uint8)).astype(bool)
        assert np.array_equal(host_bits(b_).view(np.uint8)[valid], tiled_ref(_bytes_of_bf16(a, N, cols))[valid])


# ----------------------------------------------------------------------------- the FP8 backward on tiled operands

@pytest.mark.gpu
@pytest.mark.parametrize("rows,cols,ld_out", [(64, 128, 128), (300, 512, 384), (1000, 384, 1024)])
@pytest.mark.parametrize("e5", [False, True])
def test_tiled_transposes_are_the_row_major_ones_moved(B, rows, cols, ld_out, e5):
    say(f"tiled transposes rows={rows} cols={cols} ld_out={ld_out} e5m2={e5}")
    E = B.FFN_E5M2 if e5 else B.FFN_E4M3
    x = dev_bf16(W.normal_bf16((rows, cols), 1.0, rows + cols, 31))
    am = dev_f32([3.0])
    qt1, q1, s1 = empty_u8(cols, ld_out), empty_u8(rows, cols), empty_f32(1)
    B.ffn_quant_transpose(qt1, q1, s1, x, am, rows, cols, ld_out, code_dtype=E)
    qt2 = empty_u8(B.ffn_tile_bytes(cols, ld_out)).fill_(0xA5)
    q2 = empty_u8(B.ffn_tile_bytes(rows, cols)).fill_(0xA5)
    s2, clear = empty_f32(1), dev_f32([9.0])
    B.ffn_quant_transpose_tiled(qt2, q2, s2, x, am, clear, rows, cols, ld_out, code_dtype=E)
    codes = dev_u8(_codes((rows, cols), rows))
    t1 = empty_u8(cols, ld_out)
    B.ffn_transpose(t1, codes, rows, cols, ld_out, 1)
    t2 = empty_u8(B.ffn_tile_bytes(cols, ld_out)).fill_(0xA5)
    B.ffn_transpose_tiled(t2, codes, rows, cols, ld_out)
    torch.cuda.synchronize()
    for got, want, r, c in ((qt2, qt1, cols, ld_out), (q2, q1, rows, cols), (t2, t1, cols, ld_out)):
        valid = tiled_ref(np.ones((r, c), np.uint8)).astype(bool)
        g = host_u8(got)
        assert np.array_equal(g[valid], tiled_ref(host_u8(want).reshape(r, c))[valid])
        assert np.all(g[~valid] == 0xA5)
    assert torch.equal(s1, s2) and clear.item() == 0.0


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (1000, 1024, 640), (8192, 3584, 8192)])
@pytest.mark.parametrize("e5", [False, True])
def test_tiled_tn_products_equal_the_row_major_ones(B, M, N, K, e5):
    """The backward's products on tiled operands: plain, accumulating and with
    the SwiGLU backward in the epilogue, e4m3 or e5m2 gradient codes."""
    say(f"tiled TN M={M} N={N} K={K} e5m2={e5}")
    E = B.FFN_E5M2 if e5 else B.FFN_E4M3
    a = _codes((M, K), M + 1, top=0x50)
    b = _codes((N, K), N + 2, top=0x50)
    ad, bd = dev_u8(a), dev_u8(b)
    at, bt = _pack(B, ad, M, K), _pack(B, bd, N, K)
    sa, sb = dev_f32([0.02]), dev_f32([0.03])
    T = B.FFN_TN_TILED
    o1, o2 = empty_bf16(M, N), empty_bf16(M, N)
    B.ffn_matmul_tn(o1, ad, sa, bd, sb, E, 0, M, N, K)
    B.ffn_matmul_tn(o2, at, sa, bt, sb, E, T, M, N, K)
    acc0 = dev_bf16(W.normal_bf16((M, N), 1.0, M + N, 33))
    c1, c2 = acc0.clone(), acc0.clone()
    B.ffn_matmul_tn(c1, ad, sa, bd, sb, E, B.FFN_TN_ACCUMULATE, M, N, K)
    B.ffn_matmul_tn(c2, at, sa, bt, sb, E, B.FFN_TN_ACCUMULATE | T | B.FFN_TN_TILE_GRID, M, N, K)
    gu = dev_bf16(W.normal_bf16((M, 2 * N), 1.0, M + 2 * N, 34))
    d1, d2 = empty_bf16(M, 2 * N), empty_bf16(M, 2 * N)
    m1, m2 = empty_f32(1), empty_f32(1)
    B.ffn_matmul_tn_swiglu_bwd(d1, m1, ad, sa, bd, sb, gu, E, M, N, K)
    B.ffn_matmul_tn_swiglu_bwd(d2, m2, at, sa, bt, sb, gu, E, M, N, K, flags=T)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, c2)
    assert torch.equal(d1, d2) and torch.equal(m1, m2)


@pytest.mark.gpu
@pytest.mark.parametrize("N,C,H,gd,zo,conc", [(300, 512, 384, "e4m3", True, False), (300, 512, 384, "e5m2", False, False),
                                              (1000, 1024, 1536, "e4m3", True, True),
                                              (8192, 3584, 18944, "e4m3", True, False)])
def test_tiled_backward_equals_the_row_major_backward(blk, B, N, C, H, gd, zo, conc):
    """BackwardBlock(tiled=True): gradients, scales and abs-max words equal the
    row-major backward's bit for bit, over two calls (the weight gradients
    accumulate)."""
    say(f"tiled backward N={N} C={C} H={H} grad={gd} zero_once={zo} concurrent={conc}")
    d = W.block_inputs(N, C, H, seed=N + 11)
    inp, add = dev_bf16(d["inp"]), dev_bf16(d["addend"])
    dout = dev_bf16(W.normal_bf16((N, C), 0.01, N + 12, 35))
    res = {}
    for tiled in (False, True):
        f = blk.PrefillBlock(N, C, H, 1e-5, True)
        f.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
        bb = blk.BackwardBlock(f, in_place=False, grad_dtype=gd, concurrent=conc, zero_once=zo, tiled=tiled)
        outs = []
        for rep in range(2):
            bb.forward(inp, add)
            d_res = bb.backward(dout if rep == 0 else dout * 0.5).clone()
            outs.append((d_res, bb.dgu.clone(), bb.s_dout.clone(), bb.s_dgu.clone(), bb.am_dres.clone()))
        res[tiled] = (outs, bb.dw_d.clone(), bb.dw_gu.clone(), bb.dw_norm.clone())
    torch.cuda.synchronize()
    (o0, a0, g0, n0), (o1, a1, g1, n1) = res[False], res[True]
    assert torch.equal(a0, a1) and torch.equal(g0, g1) and torch.equal(n0, n1)
    for x0, x1 in zip(o0, o1):
        for t0, t1 in zip(x0, x1):
            assert torch.equal(t0, t1)


@pytest.mark.gpu
@pytest.mark.parametrize("e5", [False, True])
def test_tiled_swiglu_bwd_rows_past_n_do_not_matter(B, e5):
    """The SwiGLU-backward epilogue on tiled operands: padding rows of the
    gradient codes that decode to NaN or infinity (e4m3 0x7F, e5m2 0x7C..0x7F)
    change neither dgu nor its abs-max."""
    M, H, K = 100, 256, 256
    say(f"tiled swiglu bwd pad rows e5m2={e5}")
    E = B.FFN_E5M2 if e5 else B.FFN_E4M3
    a = _codes((M, K), 7, top=0x40)
    bt = _pack(B, dev_u8(_codes((H, K), 8, top=0x40)), H, K)
    sa, sb = dev_f32([0.02]), dev_f32([0.02])
    gu = dev_bf16(W.normal_bf16((M, 2 * H), 1.0, 9, 36))
    res = []
    for fill in (0x00, 0x7F, 0x7C):
        pad = np.full((128, K), fill, np.uint8)
        pad[:M] = a
        at = empty_u8(B.ffn_tile_bytes(M, K))
        B.ffn_tile_pack(at, dev_u8(pad), 128, K)
        dgu, am = empty_bf16(M, 2 * H), empty_f32(1)
        B.ffn_matmul_tn_swiglu_bwd(dgu, am, at, sa, bt, sb, gu, E, M, H, K, flags=B.FFN_TN_TILED)
        res.append((dgu, am))
    torch.cuda.synchronize()
    for dgu, am in res[1:]:
        assert torch.equal(dgu, res[0][0]) and torch.equal(am, res[0][1]) and np.isfinite(am.item())
