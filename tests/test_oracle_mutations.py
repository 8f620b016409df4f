"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutation replaces one oracle function by a plausible wrong version (a
dropped term, a wrong constant, a transposed operand, a wrong rounding) and
runs the pins that should notice it.
"""

import numpy as np
import pytest

import oracle as O
import oracle.bitlinear_oracle as B
from tests import test_oracle_pins as P


def _gamma_no_abs(w):
    a = np.asarray(w, dtype=np.float64).ravel()
    return np.float32(max(np.float32(np.mean(a)), B.EPS_W))


def _gamma_max(w):
    return np.float32(np.max(np.abs(np.asarray(w, dtype=np.float64))))


def _codes_threshold_gamma(w, gamma):
    w = np.asarray(w, dtype=np.float64)
    return np.where(np.abs(w) > gamma, np.sign(w), 0).astype(np.int8)


def _codes_round_half_up(w, gamma):
    q = np.floor(np.asarray(w, dtype=np.float64) / np.float64(gamma) + 0.5)
    return np.clip(q, -1, 1).astype(np.int8)


def _pack_msb_first(q, Kp=None):
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    Kp = B.k_pad(K) if Kp is None else Kp
    full = np.zeros((N, Kp), dtype=np.int64)
    full[:, :K] = q
    f = (full & 3).reshape(N, Kp // 4, 4)
    return (f[..., 3] | (f[..., 2] << 2) | (f[..., 1] << 4) | (f[..., 0] << 6)).astype(np.uint8)


def _act_128(x, Kp=None):
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    Kp = B.k_pad(K) if Kp is None else Kp
    s = np.maximum(np.max(np.abs(x), axis=1).astype(np.float32), B.EPS_X)
    q = np.clip(np.rint(128.0 * x / s[:, None]), -127, 127)
    out = np.zeros((M, Kp), dtype=np.int8)
    out[:, :K] = q
    return out, s


def _act_trunc(x, Kp=None):
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    Kp = B.k_pad(K) if Kp is None else Kp
    s = np.maximum(np.max(np.abs(x), axis=1).astype(np.float32), B.EPS_X)
    q = np.clip(np.trunc(127.0 * x / s[:, None]), -127, 127)
    out = np.zeros((M, Kp), dtype=np.int8)
    out[:, :K] = q
    return out, s


def _y_no_127(acc, s, gamma):
    return np.asarray(acc, np.float64) * np.asarray(s, np.float64)[:, None] * np.float64(gamma)


def _backward_dw_swapped(dY, x_q, s, q, gamma):
    K = np.asarray(q).shape[1]
    dY = np.asarray(dY, dtype=np.float64)
    xh = B.x_hat(x_q, s, K)
    dX = dY @ B.w_hat(q, gamma)
    dW = (dY.T @ xh)[::-1]  # rows of dW in the wrong order
    return dX, dW


def _backward_dx_fp32_gamma(dY, x_q, s, q, gamma):
    K = np.asarray(q).shape[1]
    dY = np.asarray(dY, dtype=np.float64)
    dX = dY @ (np.asarray(q, np.float64) * np.float64(gamma))  # bf16(gamma) dropped
    dW = dY.T @ B.x_hat(x_q, s, K)
    return dX, dW


def _xhat_unrounded(x_q, s, K):
    return np.asarray(x_q)[:, :K].astype(np.float64) * np.asarray(s, np.float64)[:, None] / 127.0


def _bf16_trunc(v):
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def _sign1_msb_first(dW, Kp=None):
    d = np.asarray(dW, dtype=np.float64)
    N, K = d.shape
    Kp = B.k_pad(K) if Kp is None else Kp
    neg = np.zeros((N, Kp), dtype=np.int64)
    neg[:, :K] = d < 0
    bits = neg.reshape(N, Kp // 8, 8)
    out = np.zeros((N, Kp // 8), dtype=np.int64)
    for j in range(8):
        out |= bits[..., j] << (7 - j)
    return out.astype(np.uint8)


def _sign1_zero_negative(dW, Kp=None):
    d = np.asarray(dW, dtype=np.float64)
    return _sign1_ref(np.where(d <= 0, -1.0, 1.0), Kp)


def _sign1_inverted(dW, Kp=None):
    return _sign1_ref(-np.asarray(dW, dtype=np.float64), Kp)


_sign1_ref = B.sign1_pack


def _bias_grad_rows(dY):
    d = np.asarray(dY, dtype=np.float64)
    return d.sum(axis=1)[: d.shape[1]] if d.shape[0] >= d.shape[1] else np.resize(d.sum(axis=1), d.shape[1])


def _forward_y_bias_minus(acc, s, gamma, bias):
    return B.forward_y(acc, s, gamma) - np.asarray(bias, dtype=np.float64)[None, :]


MUTATIONS = [
    ("absmean_gamma", _gamma_no_abs, ["test_gamma_closed_forms", "test_codes_zero_fraction_statistics"]),
    ("absmean_gamma", _gamma_max, ["test_gamma_closed_forms", "test_codes_zero_fraction_statistics"]),
    ("ternary_codes", _codes_threshold_gamma, ["test_codes_hand_examples_and_ties", "test_codes_vs_fraction_bruteforce"]),
    ("ternary_codes", _codes_round_half_up, ["test_codes_hand_examples_and_ties", "test_codes_vs_fraction_bruteforce"]),
    ("pack_codes", _pack_msb_first, ["test_pack_hand_bytes"]),
    ("act_quant", _act_128, ["test_act_quant_invariants", "test_act_quant_exhaustive_bf16_significands"]),
    ("act_quant", _act_trunc, ["test_act_quant_vs_fraction_and_ties", "test_act_quant_exhaustive_bf16_significands"]),
    ("forward_y", _y_no_127, ["test_y_dx_dw_exact_fractions", "test_against_torch_autograd_detach_ste"]),
    ("backward", _backward_dw_swapped, ["test_backward_one_hot_dY_selects_rows", "test_y_dx_dw_exact_fractions"]),
    ("backward", _backward_dx_fp32_gamma, ["test_y_dx_dw_exact_fractions", "test_against_torch_autograd_detach_ste"]),
    ("x_hat", _xhat_unrounded, ["test_y_dx_dw_exact_fractions"]),
    ("bf16_round", _bf16_trunc, ["test_bf16_round_matches_exact_rounding", "test_bf16_bits_roundtrip"]),
    ("sign1_pack", _sign1_msb_first, ["test_sign1_hand_bytes", "test_sign1_matches_numpy_packbits"]),
    ("sign1_pack", _sign1_zero_negative, ["test_sign1_hand_bytes", "test_sign1_matches_numpy_packbits"]),
    ("sign1_pack", _sign1_inverted, ["test_sign1_hand_bytes", "test_sign1_of_ste_gradient_matches_quantised_gradient"]),
    ("bias_grad", _bias_grad_rows, ["test_bias_grad_exact_column_sums", "test_bias_against_torch_autograd"]),
    ("forward_y_bias", _forward_y_bias_minus, ["test_bias_against_torch_autograd"]),
]


@pytest.mark.parametrize("name,fn,pins", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    monkeypatch.setattr(B, name, fn)
    monkeypatch.setattr(O, name, fn)
    caught = []
    for pin in pins:
        try:
            getattr(P, pin)()
        except (AssertionError, ValueError):
            caught.append(pin)
    assert caught, f"mutation {fn.__name__} of {name} passed every pin in {pins}"


# ---------------------------------------------------------------------------
# TTQ oracle
# ---------------------------------------------------------------------------

import math  # noqa: E402

import oracle.ttq_oracle as T  # noqa: E402


def _ttq_codes_inclusive(w, delta):
    w = np.asarray(w, dtype=np.float64)
    d = np.float64(delta)
    return np.where(w >= d, 1, np.where(w <= -d, -1, 0)).astype(np.int8)


def _ttq_init_half(w):
    e = B.absmean_gamma(w)
    return np.float32(0.5 * e), np.float32(e), np.float32(e)


def _ttq_values_swapped(q, wp, wn):
    q = np.asarray(q)
    p = B.bf16_round(np.float64(wn))
    n = B.bf16_round(np.float64(wp))
    return np.where(q == 1, p, np.where(q == -1, -n, 0.0))


def _ttq_values_unrounded(q, wp, wn):
    q = np.asarray(q)
    return np.where(q == 1, np.float64(wp), np.where(q == -1, -np.float64(wn), 0.0))


def _ttq_backward_wn_sign(dY, x, q, wp, wn):
    dX, dW, g_wp, g_wn = _ttq_backward_ref(dY, x, q, wp, wn)
    return dX, dW, g_wp, -g_wn


def _ttq_backward_wp_all_nonzero(dY, x, q, wp, wn):
    dX, dW, g_wp, g_wn = _ttq_backward_ref(dY, x, q, wp, wn)
    return dX, dW, math.fsum(dW[np.asarray(q) != 0].tolist()), g_wn


def _ttq_backward_dx_unsigned(dY, x, q, wp, wn):
    dX, dW, g_wp, g_wn = _ttq_backward_ref(dY, x, q, wp, wn)
    return np.asarray(dY, np.float64) @ np.abs(T.ttq_values(q, wp, wn)), dW, g_wp, g_wn


def _ttq_backward_dw_scaled(dY, x, q, wp, wn):
    # the paper's scaled gradient instead of the page's identity STE
    dX, dW, g_wp, g_wn = _ttq_backward_ref(dY, x, q, wp, wn)
    q = np.asarray(q)
    s = np.where(q == 1, np.float64(wp), np.where(q == -1, np.float64(wn), 1.0))
    return dX, dW * s, g_wp, g_wn


_ttq_backward_ref = T.ttq_backward

TTQ_MUTATIONS = [
    ("ttq_codes", _ttq_codes_inclusive, ["test_ttq_codes_strict_threshold", "test_ttq_reduces_to_bitnet_quantizer"]),
    ("ttq_init", _ttq_init_half, ["test_ttq_init_hand_example", "test_ttq_init_is_point_seven_of_mean_abs"]),
    ("ttq_values", _ttq_values_swapped, ["test_ttq_values_hand", "test_ttq_against_torch_autograd"]),
    ("ttq_values", _ttq_values_unrounded, ["test_ttq_values_hand", "test_ttq_reduces_to_bitnet_quantizer"]),
    ("ttq_backward", _ttq_backward_wn_sign, ["test_ttq_against_torch_autograd", "test_ttq_grads_exact_fractions"]),
    ("ttq_backward", _ttq_backward_wp_all_nonzero, ["test_ttq_against_torch_autograd", "test_ttq_grads_exact_fractions"]),
    ("ttq_backward", _ttq_backward_dx_unsigned, ["test_ttq_against_torch_autograd", "test_ttq_grads_exact_fractions"]),
    ("ttq_backward", _ttq_backward_dw_scaled, ["test_ttq_against_torch_autograd", "test_ttq_grads_exact_fractions"]),
]


@pytest.mark.parametrize("name,fn,pins", TTQ_MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in TTQ_MUTATIONS])
def test_planted_ttq_mistake_is_caught(monkeypatch, name, fn, pins):
    monkeypatch.setattr(T, name, fn)
    monkeypatch.setattr(O, name, fn)
    caught = []
    for pin in pins:
        try:
            getattr(P, pin)()
        except (AssertionError, ValueError):
            caught.append(pin)
    assert caught, f"mutation {fn.__name__} of {name} passed every pin in {pins}"


# ---------------------------------------------------------------------------
# the parity gate (oracle/compare.py) and the sampled TTQ references
# ---------------------------------------------------------------------------

import oracle.compare as CMP  # noqa: E402
from tests import test_compare_pins as CP  # noqa: E402

_check_ref = CMP.check
_rel_errors_ref = CMP.rel_errors


def _check_always_floors(got, ref, what):
    m = _rel_errors_ref(got, ref, 2.0 ** -8)
    assert m["max_rel"] <= CMP.MAX_REL, (what, m)
    assert m["normwise"] <= CMP.NORMWISE, (what, m)
    return m


def _check_no_normwise(got, ref, what):
    m = _rel_errors_ref(got, ref, 0.0 if what == "y" else 2.0 ** -8)
    assert m["max_rel"] <= CMP.MAX_REL, (what, m)
    return m


def _check_mean_rel(got, ref, what):
    # the mean instead of the maximum of the element errors
    m = dict(_rel_errors_ref(got, ref, 0.0 if what == "y" else 2.0 ** -8))
    g = np.asarray(got, np.float64)
    o = np.asarray(ref, np.float64)
    m["max_rel"] = float(np.mean(np.abs(g - o) / np.maximum(np.abs(o), 1e-300)))
    assert m["max_rel"] <= CMP.MAX_REL, (what, m)
    assert m["normwise"] <= CMP.NORMWISE, (what, m)
    return m


def _rel_errors_zero_over_zero(got, ref, floor_frac):
    # 0/0 taken as an error instead of an exact match
    m = dict(_rel_errors_ref(got, ref, floor_frac))
    g = np.asarray(got, np.float64)
    o = np.asarray(ref, np.float64)
    if np.any((g == o) & (o == 0)) and floor_frac == 0:
        m["max_rel"] = float("inf")
    return m


def _rel_errors_nan_ignored(got, ref, floor_frac):
    g = np.asarray(got, np.float64)
    o = np.asarray(ref, np.float64)
    ok = np.isfinite(g)
    return _rel_errors_ref(g[ok], o[ok], floor_frac)


def _near_w_off_by_gamma(w, gamma):
    # the boundary taken at gamma instead of gamma / 2
    h = np.float32(gamma)
    a = np.abs(np.asarray(w, dtype=np.float64))
    return int(np.sum(np.abs(a - np.float64(h)) <= np.float64(np.spacing(h))))


def _near_a_integers(x, s):
    # integers instead of half-integers
    t = 127.0 * np.asarray(x, np.float64) / np.asarray(s, np.float64)[:, None]
    ulp = np.spacing(np.abs(t).astype(np.float32)).astype(np.float64)
    return int(np.sum(np.abs(t - np.rint(t)) <= ulp))


def _ttq_dx_elements_transposed(dY, wt, rows, cols):
    dY = np.asarray(dY, dtype=np.float64)
    wt = np.asarray(wt, dtype=np.float64)
    return np.array([float(np.dot(dY[m], wt[k])) for m, k in zip(rows, cols)])


def _ttq_dw_elements_swapped(dY, x, rows, cols):
    dY = np.asarray(dY, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return np.array([float(np.dot(dY[:, k], x[:, n])) for n, k in zip(rows, cols)])


def _ttq_y_elements_transposed(x, wt, rows, cols):
    x = np.asarray(x, dtype=np.float64)
    wt = np.asarray(wt, dtype=np.float64)
    return np.array([float(np.dot(x[m], wt[:, n])) for m, n in zip(rows, cols)])


_SQ = dict(M=6, N=6, K=6)
GATE_MUTATIONS = [
    (CMP, "check", _check_always_floors, [("test_y_has_no_floor", {}), ("test_floored_kinds_use_the_floor", {})]),
    (CMP, "check", _check_no_normwise, [("test_uniform_normwise_offset_fails", {})]),
    (CMP, "check", _check_mean_rel, [("test_one_element_off_by_one_percent_fails", {})]),
    (CMP, "rel_errors", _rel_errors_zero_over_zero, [("test_exact_match_and_zeros_pass", {})]),
    (CMP, "rel_errors", _rel_errors_nan_ignored, [("test_nan_and_inf_fail", {})]),
    (CMP, "near_boundary_weights", _near_w_off_by_gamma, [("test_near_boundary_weights_hand_count", {})]),
    (CMP, "near_boundary_acts", _near_a_integers, [("test_near_boundary_acts_hand_count", {}),
                                                   ("test_near_boundary_acts_zero_is_not_a_boundary", {})]),
    (T, "ttq_dx_elements", _ttq_dx_elements_transposed, [("test_ttq_element_helpers_match_full_functions", _SQ),
                                                        ("test_ttq_element_helpers_hand_values", {})]),
    (T, "ttq_dw_elements", _ttq_dw_elements_swapped, [("test_ttq_element_helpers_match_full_functions", _SQ),
                                                     ("test_ttq_element_helpers_hand_values", {})]),
    (T, "ttq_y_elements", _ttq_y_elements_transposed, [("test_ttq_element_helpers_match_full_functions", _SQ),
                                                      ("test_ttq_element_helpers_hand_values", {})]),
]


@pytest.mark.parametrize("mod,name,fn,pins", GATE_MUTATIONS, ids=[f"{m[1]}:{m[2].__name__}" for m in GATE_MUTATIONS])
def test_planted_gate_mistake_is_caught(monkeypatch, mod, name, fn, pins):
    monkeypatch.setattr(mod, name, fn)
    if hasattr(O, name):
        monkeypatch.setattr(O, name, fn)
    caught = []
    for pin, kw in pins:
        try:
            getattr(CP, pin)(**kw)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin)
        except BaseException as e:  # pytest.raises(...) not raised is a Failed, not an AssertionError
            if type(e).__name__ == "Failed":
                caught.append(pin)
            else:
                raise
    assert caught, f"mutation {fn.__name__} of {name} passed every pin in {[p for p, _ in pins]}"
