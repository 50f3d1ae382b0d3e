"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin
catches each one.  This shows the pins are tight enough to matter."""

import numpy as np
import pytest

import oracle
import oracle.ffn as OF
from oracle import codecs as K
from tests import test_oracle_codecs as TC
from tests import test_oracle_ffn as TF


def _fails(fn):
    with pytest.raises(AssertionError):
        fn()


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(OF, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def test_swapped_gate_and_up_is_caught(monkeypatch):
    good = OF.swiglu

    def swapped(gu_bits):
        H = gu_bits.shape[-1] // 2
        return good(np.concatenate([gu_bits[..., H:], gu_bits[..., :H]], axis=-1))
    _patch(monkeypatch, "swiglu", swapped)
    _fails(TF.test_swiglu_gate_up_placement_and_torch)


def test_dropped_eps_is_caught(monkeypatch):
    good = OF.rmsnorm_fwd
    _patch(monkeypatch, "rmsnorm_fwd", lambda a, b, w, eps: good(a, b, w, 0.0))
    _fails(TF.test_rmsnorm_degenerate_rows)


def test_mean_by_wrong_count_is_caught(monkeypatch):
    good = OF.rmsnorm_fwd

    def bad(a, b, w, eps):
        r, y, rstd, am = good(a, b, w, eps)
        return r, y, (rstd * np.float32(1.0001)).astype(np.float32), am
    _patch(monkeypatch, "rmsnorm_fwd", bad)
    _fails(TF.test_rmsnorm_matches_torch_rms_norm)


def test_wrong_silu_sign_is_caught(monkeypatch):
    _patch(monkeypatch, "silu", lambda g: np.asarray(g, np.float64) / (1.0 + np.exp(np.asarray(g, np.float64))))
    _fails(TF.test_silu_closed_forms_and_torch)


def test_quantising_with_scale_instead_of_inverse_is_caught(monkeypatch):
    def bad(x_bits, absmax=None):
        if absmax is None:
            absmax = OF.absmax_of(x_bits)
        scale, inv = OF.scales_from_absmax(absmax)
        q = K.e4m3_encode(K.bf16_bits_to_f64(x_bits).astype(np.float32) * scale)
        return q, scale, np.float32(absmax)
    _patch(monkeypatch, "quant_absmax", bad)
    _fails(TF.test_quant_matches_torch_float8)


def test_weight_read_in_the_wrong_layout_is_caught(monkeypatch):
    # reading the [O, K] weight as if it were stored [K, O]
    monkeypatch.setattr(OF, "_matmul_nt", lambda x, w: np.asarray(x, np.float64)
                        @ np.asarray(w, np.float64).reshape(w.shape[1], w.shape[0]))
    _fails(TF.test_gemm_bf16_brute_force_exact_fractions)


def test_missing_scale_product_is_caught(monkeypatch):
    def bad(qx, sx, qw, sw):
        return K.f64_to_bf16_bits(OF._matmul_nt(K.e4m3_decode(qx), K.e4m3_decode(qw)) * np.float64(sx))
    _patch(monkeypatch, "gemm_fp8", bad)
    _fails(TF.test_gemm_fp8_matches_torch_and_scales)


def test_e4m3_ties_away_from_zero_is_caught(monkeypatch):
    good = K.e4m3_encode

    def bad(v):
        v = np.asarray(v, np.float64)
        return good(v + np.copysign(1e-12, v) * np.abs(v))
    monkeypatch.setattr(K, "e4m3_encode", bad)
    _fails(TC.test_e4m3_encode_brute_force)


def test_bf16_truncation_is_caught(monkeypatch):
    def trunc(v):
        v = np.asarray(v, np.float64).astype(np.float32)
        return ((v.view(np.uint32) >> 16) << 16).view(np.float32).astype(np.float64)
    monkeypatch.setattr(K, "bf16_round", trunc)
    _fails(TC.test_bf16_round_of_float64_by_nearest_search)


# ----------------------------------------------------------------------------- backward

import oracle.backward as OB
from tests import test_oracle_backward as TB


def _patch_b(monkeypatch, name, fn):
    monkeypatch.setattr(OB, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def test_swapped_gate_and_up_gradients_are_caught(monkeypatch):
    good = OB.swiglu_bwd

    def swapped(dh, gu):
        dgu, am = good(dh, gu)
        H = dgu.shape[-1] // 2
        return np.concatenate([dgu[..., H:], dgu[..., :H]], axis=-1), am
    _patch_b(monkeypatch, "swiglu_bwd", swapped)
    _fails(TB.test_swiglu_bwd_matches_torch_autograd)
    _fails(TB.test_block_backward_zero_gate_and_accumulators)


def test_silu_derivative_without_its_second_term_is_caught(monkeypatch):
    def bad(dh_bits, gu_bits):
        dh, gu = K.bf16_bits_to_f64(dh_bits), K.bf16_bits_to_f64(gu_bits)
        H = gu.shape[-1] // 2
        g, u = gu[..., :H], gu[..., H:]
        s = OB.sigmoid(g)
        dgu = np.concatenate([K.bf16_round(dh * u * s), K.bf16_round(dh * g * s)], axis=-1)
        return K.f64_to_bf16_bits(dgu), np.float32(np.max(np.abs(dgu)))
    _patch_b(monkeypatch, "swiglu_bwd", bad)
    _fails(TB.test_swiglu_bwd_finite_differences)
    _fails(TB.test_swiglu_bwd_matches_torch_autograd)


def test_rmsnorm_backward_without_the_normalisation_term_is_caught(monkeypatch):
    good = OB.rmsnorm_bwd

    def bad(dres, dy, r, w, rstd, dweight=None):
        _, dw, _ = good(dres, dy, r, w, rstd, dweight)
        rs = np.asarray(rstd, np.float32).astype(np.float64)[..., None]
        dinp = K.bf16_round(K.bf16_bits_to_f64(dres) + rs * K.bf16_bits_to_f64(dy) * K.bf16_bits_to_f64(w)[None, :])
        return K.f64_to_bf16_bits(dinp), dw, np.float32(np.max(np.abs(dinp)))
    _patch_b(monkeypatch, "rmsnorm_bwd", bad)
    _fails(TB.test_rmsnorm_bwd_matches_torch_autograd)
    _fails(TB.test_rmsnorm_bwd_is_orthogonal_to_the_input_without_eps)
    _fails(lambda: TB.test_block_backward_matches_torch_autograd(False))


def test_weight_gradient_without_accumulation_is_caught(monkeypatch):
    good = OB.matmul_tn
    _patch_b(monkeypatch, "matmul_tn", lambda a, b, a_scale=None, b_scale=None, accumulate=None:
             good(a, b, a_scale, b_scale))
    _fails(TB.test_matmul_tn_and_accumulate)
    _fails(TB.test_linear_bwd_bf16_matches_torch_autograd)


def test_fp8_gradient_scaled_by_the_input_scale_is_caught(monkeypatch):
    good = OB.linear_bwd

    def bad(dy, x, w, fp8=False, dy_absmax=None, qx=None, sx=None, qw=None, sw=None, dw_acc=None):
        out = good(dy, x, w, fp8, dy_absmax, qx, sx, qw, sw, dw_acc)
        if fp8:
            out["dx"] = OB.matmul_tn(out["qdy"], OB.transpose(qw), sx, sw)
        return out
    _patch_b(monkeypatch, "linear_bwd", bad)
    _fails(TB.test_linear_bwd_fp8_scales_exactly_with_the_gradient)
