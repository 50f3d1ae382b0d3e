"""Pins for the oracle's number formats (bf16, OCP e4m3fn).

Each check ties the oracle to something other than itself: torch's own CPU
conversions (an independent library), brute-force nearest-value search over
all codes, and the closed-form landmarks of the formats.
"""

import numpy as np
import pytest
import torch

from oracle import codecs as K

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _all_bf16():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _torch_bf16_bits(x_f32):
    return torch.from_numpy(np.asarray(x_f32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- bf16

def test_bf16_exhaustive_round_trip():
    bits = _all_bf16()
    v = K.bf16_bits_to_f64(bits)
    back = K.f64_to_bf16_bits(v)
    finite = ~np.isnan(v)
    assert np.array_equal(back[finite], bits[finite])
    assert np.all(np.isnan(K.bf16_bits_to_f64(back[~finite])))


def test_bf16_encode_matches_torch_on_random_and_edge_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),  # bf16 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32),
    ])
    # exact ties: a bf16 value plus half an ulp (bit 15 set, low bits clear)
    ties = ((rng.integers(0, 65536, 50_000, dtype=np.uint32) << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    got = K.f64_to_bf16_bits(x.astype(np.float64))
    want = _torch_bf16_bits(x)
    assert np.array_equal(got, want)


def test_bf16_round_of_float64_by_nearest_search():
    # float64 inputs that float32 cannot hold: compare with the nearest finite
    # bf16 value found by search over the sorted table (ties -> even pattern).
    bits = _all_bf16()
    vals = K.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals) & ~((vals == 0) & (bits == 0x8000))
    vals, bits = vals[keep], bits[keep]
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20_000) * np.exp(rng.uniform(-20, 20, 20_000))
    x = np.concatenate([x, (vals[1000:1100] + vals[1001:1101]) / 2])  # exact midpoints
    i = np.clip(np.searchsorted(vals, x), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = x - lo, hi - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((bits[i] & 1) == 0))
    want = np.where(pick_hi, hi, lo)
    assert np.array_equal(K.bf16_round(x), want)


def test_bf16_landmarks():
    assert K.bf16_bits_to_f64(np.array([0x3F80]))[0] == 1.0
    assert K.bf16_bits_to_f64(np.array([0x7F7F]))[0] == K.BF16_MAX
    assert K.f64_to_bf16_bits(np.array([1.0 + 2 ** -8]))[0] == 0x3F80      # tie -> even
    assert K.f64_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82  # tie -> even (up)
    assert K.f64_to_bf16_bits(np.array([-0.0]))[0] == 0x8000


# ----------------------------------------------------------------------------- e4m3

def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = K.e4m3_decode(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}


def test_e4m3_format_landmarks():
    fi = torch.finfo(torch.float8_e4m3fn)
    d = K.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.nanmax(d) == K.E4M3_MAX == fi.max == 448.0
    assert d[0x08] == fi.smallest_normal == 2.0 ** -6
    assert d[0x01] == 2.0 ** -9
    assert d[0x38] == 1.0 and d[0xB8] == -1.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    # 254 finite codes, 253 distinct values (+0 and -0 coincide)
    assert np.isfinite(d).sum() == 254 and len(np.unique(d[np.isfinite(d)])) == 253


def _brute_e4m3(x):
    """Nearest finite code by exhaustive search; ties to the code with an even
    mantissa; |x| >= 448 saturates; the sign of zero is kept."""
    codes = np.arange(256, dtype=np.int64)
    vals = K.e4m3_decode(codes.astype(np.uint8))
    fin = np.isfinite(vals)
    codes, vals = codes[fin], vals[fin]
    out = np.empty(x.shape, np.uint8)
    for idx, v in enumerate(x):
        a = min(abs(v), 448.0)
        pos = codes < 128
        d = np.abs(vals[pos] - a)
        best = np.flatnonzero(d == d.min())
        cand = codes[pos][best]
        if len(cand) > 1:
            cand = cand[(cand & 1) == 0]
        c = int(cand[0])
        if np.signbit(v):
            c |= 0x80
        out[idx] = c
    return out


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(11)
    vals = K.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([
        rng.standard_normal(3000) * np.exp(rng.uniform(-8, 6.5, 3000)),
        mids, -mids, vals, -vals,
        [0.0, -0.0, 448.0, 460.0, 464.0, 500.0, -1e9, 2.0 ** -10, 2.0 ** -10 * 3, 2.0 ** -11],
    ])
    assert np.array_equal(K.e4m3_encode(x), _brute_e4m3(x))


def test_e4m3_encode_matches_torch_on_all_bf16_times_scales():
    bits = _all_bf16()
    x = K.bf16_bits_to_f64(bits).astype(np.float32)
    x = x[np.isfinite(x)]
    for inv in [1.0, 0.37, 3.1, 279.72677, 1.0 / 448.0, 448.0 / 7.5]:
        p = x * np.float32(inv)
        p = p[np.isfinite(p)]
        want = torch.from_numpy(np.clip(p, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = K.e4m3_encode(p)
        assert np.array_equal(got, want), inv


def test_e4m3_encode_special_values():
    assert K.e4m3_encode(np.array([np.nan]))[0] == 0x7F
    assert K.e4m3_encode(np.array([-np.nan]))[0] == 0xFF
    assert K.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert K.e4m3_encode(np.array([1e30]))[0] == 0x7E
    assert K.e4m3_encode(np.array([-np.inf]))[0] == 0xFE
    # subnormal grid 2^-9 with ties to even: 0.5 ulp -> 0, 1.5 ulp -> 2, 2.5 -> 2
    s = 2.0 ** -9
    assert list(K.e4m3_encode(np.array([0.5 * s, 1.5 * s, 2.5 * s, 7.5 * s]))) == [0, 2, 2, 8]


# ----------------------------------------------------------------------------- e5m2

def test_e5m2_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = K.e5m2_decode(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])          # includes +-inf at 0x7C / 0xFC
    assert set(np.flatnonzero(nan)) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}


def test_e5m2_format_landmarks():
    fi = torch.finfo(torch.float8_e5m2)
    d = K.e5m2_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(d)
    assert np.max(d[fin]) == K.E5M2_MAX == fi.max == 57344.0
    assert d[0x04] == fi.smallest_normal == 2.0 ** -14
    assert d[0x01] == 2.0 ** -16
    assert d[0x3C] == 1.0 and d[0xBC] == -1.0
    assert d[0x7B] == 57344.0 and d[0xFB] == -57344.0
    assert d[0x7C] == np.inf and d[0xFC] == -np.inf
    assert fin.sum() == 248 and len(np.unique(d[fin])) == 247


def _brute_e5m2(x):
    """Nearest finite code by exhaustive search; ties to the code with an even
    mantissa; |x| >= 57344 saturates; the sign of zero is kept."""
    codes = np.arange(128, dtype=np.int64)
    vals = K.e5m2_decode(codes.astype(np.uint8))
    fin = np.isfinite(vals)
    codes, vals = codes[fin], vals[fin]
    out = np.empty(x.shape, np.uint8)
    for idx, v in enumerate(x):
        a = min(abs(v), K.E5M2_MAX)
        d = np.abs(vals - a)
        cand = codes[np.flatnonzero(d == d.min())]
        if len(cand) > 1:
            cand = cand[(cand & 1) == 0]
        c = int(cand[0])
        if np.signbit(v):
            c |= 0x80
        out[idx] = c
    return out


def test_e5m2_encode_brute_force():
    rng = np.random.default_rng(12)
    vals = K.e5m2_decode(np.arange(0, 0x7C, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([
        rng.standard_normal(3000) * np.exp(rng.uniform(-12, 11, 3000)),
        mids, -mids, vals, -vals,
        [0.0, -0.0, 57344.0, 61440.0, 65536.0, 1e9, -1e9, 2.0 ** -17, 3 * 2.0 ** -17, 2.0 ** -18],
    ])
    assert np.array_equal(K.e5m2_encode(x), _brute_e5m2(x))


def test_e5m2_encode_matches_torch_on_all_bf16_times_scales():
    bits = _all_bf16()
    x = K.bf16_bits_to_f64(bits).astype(np.float32)
    x = x[np.isfinite(x)]
    for inv in [1.0, 0.37, 3.1, 279.72677, 1.0 / 57344.0, 57344.0 / 7.5]:
        p = x * np.float32(inv)
        p = p[np.isfinite(p)]
        want = torch.from_numpy(np.clip(p, -57344, 57344)).to(torch.float8_e5m2).view(torch.uint8).numpy()
        got = K.e5m2_encode(p)
        assert np.array_equal(got, want), inv


def test_e5m2_encode_special_values():
    assert K.e5m2_encode(np.array([np.nan]))[0] == 0x7E
    assert K.e5m2_encode(np.array([-np.nan]))[0] == 0xFE
    assert K.e5m2_encode(np.array([-0.0]))[0] == 0x80
    assert K.e5m2_encode(np.array([1e30]))[0] == 0x7B
    assert K.e5m2_encode(np.array([-np.inf]))[0] == 0xFB
    s = 2.0 ** -16
    assert list(K.e5m2_encode(np.array([0.5 * s, 1.5 * s, 2.5 * s, 3.5 * s]))) == [0, 2, 2, 4]
