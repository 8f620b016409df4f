"""Pins of the parity gate itself (oracle/compare.py) and of the oracle's
sampled-element helpers, on the CPU.

Every GPU parity test ends in ``compare.check`` (or compares sampled elements
from the ``*_elements`` helpers), so a checker that floors where it must not,
mishandles an exact zero or ignores the normwise bar would make all of them
hollow. These tests feed it hand-built (got, ref) pairs whose metrics are known
in closed form, with the bar of the layer: max relative error <= 8e-3 and
normwise error <= 5e-3, rel = |g - o| / max(|o|, tau), tau = 0 for y and
2^-8 RMS(o) for dX and dW. The near-boundary counters (elements within one
fp32 ulp of a rounding boundary: |w| = gamma/2 for the ternary codes, a
half-integer of 127x/s for the int8 activations) get constructed inputs with
hand-counted answers.
"""

import math

import numpy as np
import pytest

import oracle as O
from oracle import compare as C


def _fails(got, ref, what):
    with pytest.raises(AssertionError):
        C.check(got, ref, what)


# ---------------------------------------------------------------------------
# rel_errors / check
# ---------------------------------------------------------------------------

def test_rel_errors_closed_form():
    """ref = [1, 2, 4], got = [1, 2.01, 4]: rel = 0.01/2 = 5e-3 at element 1,
    normwise = 0.01 / sqrt(1 + 4 + 16)."""
    m = C.rel_errors([1.0, 2.01, 4.0], [1.0, 2.0, 4.0], 0.0)
    assert m["max_rel"] == pytest.approx(0.005, rel=1e-12)
    assert m["normwise"] == pytest.approx(0.01 / math.sqrt(21.0), rel=1e-12)
    assert m["tau"] == 0.0 and m["n_below_floor"] == 0


def test_rel_errors_floor_is_fraction_of_rms():
    """tau = floor_frac * RMS(ref); elements with |ref| < tau use tau as the
    denominator and are counted, the unfloored maximum is reported too."""
    ref = np.array([3.0, -4.0, 2e-6, 1e-6])  # RMS = 2.5 to 1e-12 relative
    got = ref + np.array([0.0, 0.0, 1e-4, 1e-4])
    m = C.rel_errors(got, ref, 0.01)
    assert m["tau"] == pytest.approx(0.025, rel=1e-12)
    assert m["n_below_floor"] == 2
    assert m["max_rel"] == pytest.approx(1e-4 / 0.025, rel=1e-12)
    assert m["max_rel_unfloored"] == pytest.approx(1e-4 / 1e-6, rel=1e-9)


def test_exact_match_and_zeros_pass():
    """Identical vectors pass with zero error for every kind; 0 against 0 is
    no error (y has no floor, so this is the 0/0 case)."""
    ref = np.array([0.0, 1.5, -2.25, 0.0, 7.0])
    for what in ("y", "dX", "dW"):
        m = C.check(ref.copy(), ref, what)
        assert m["max_rel"] == 0.0 and m["normwise"] == 0.0
    m = C.check(np.zeros(4), np.zeros(4), "y")
    assert m["max_rel"] == 0.0 and m["normwise"] == 0.0


def test_one_bf16_rounding_passes():
    """A bf16 rounding of each element (relative error <= 2^-9) is inside
    the bar for y, dX and dW."""
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(4096)
    got = ref * (1.0 + 2.0 ** -9 * rng.choice([-1.0, 1.0], size=ref.size))
    for what in ("y", "dX", "dW"):
        m = C.check(got, ref, what)
        assert m["max_rel"] == pytest.approx(2.0 ** -9, rel=1e-9)


def test_one_element_off_by_one_percent_fails():
    """One element 1e-2 off (relative, where |ref| is well above the floor)
    fails y and dX and dW, even though the normwise error is tiny."""
    rng = np.random.default_rng(4)
    ref = rng.standard_normal(10000) + 3.0
    ref[1234] = 2.5
    got = ref.copy()
    got[1234] *= 1.01
    assert C.rel_errors(got, ref, 2.0 ** -8)["normwise"] < 1e-3
    for what in ("y", "dX", "dW"):
        _fails(got, ref, what)


def test_uniform_normwise_offset_fails():
    """Every element 6e-3 off: max_rel 6e-3 is inside 8e-3, but normwise
    6e-3 is outside 5e-3, so the check fails on the normwise bar."""
    ref = np.random.default_rng(5).standard_normal(1000)
    got = ref * (1.0 + 6e-3)
    m = C.rel_errors(got, ref, 0.0)
    assert m["max_rel"] == pytest.approx(6e-3, rel=1e-9) and m["normwise"] == pytest.approx(6e-3, rel=1e-9)
    for what in ("y", "dX"):
        _fails(got, ref, what)


def test_y_has_no_floor():
    """y's accumulator is exact, so an exact zero must come out as zero: a
    nonzero result where ref = 0 fails y however small it is, while dX
    (floored at 2^-8 RMS) accepts the same tiny absolute error."""
    ref = np.array([0.0, 1.0, -1.0, 2.0])
    got = ref.copy()
    got[0] = 1e-9
    _fails(got, ref, "y")
    assert C.rel_errors(got, ref, 0.0)["max_rel"] == math.inf
    m = C.check(got, ref, "dX")
    assert m["n_below_floor"] == 1 and m["max_rel"] < 1e-6


def test_nan_and_inf_fail():
    ref = np.array([1.0, 2.0, 3.0])
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[1] = bad
        for what in ("y", "dX", "dW"):
            _fails(got, ref, what)


def test_floored_kinds_use_the_floor():
    """The kinds that need the floor (fp32 sums that can cancel) accept an
    error of 1e-5 RMS at an element whose reference cancelled to ~0 (rel
    1e-5 / 2^-8 = 2.6e-3); y, which has no floor, rejects it."""
    ref = np.full(64, 1.0)
    ref[7] = 1e-12
    got = ref.copy()
    got[7] += 1e-5
    for what in ("dX", "dW", "db", "y_bias", "y_ttq"):
        C.check(got, ref, what)
    _fails(got, ref, "y")


# ---------------------------------------------------------------------------
# near-boundary counters
# ---------------------------------------------------------------------------

def test_near_boundary_weights_hand_count():
    """gamma = 1: the boundary is |w| = 0.5, whose fp32 ulp is 2^-23 * 0.5 =
    2^-24. Within it: 0.5, -0.5, 0.5 + 2^-24, 0.5 - 2^-25 (4). Outside: 0.5 +
    2^-22, 0.25, 0.75, 0."""
    u = 2.0 ** -24
    w = np.array([0.5, -0.5, 0.5 + u, 0.5 - u / 2, 0.5 + 4 * u, 0.25, 0.75, 0.0])
    assert C.near_boundary_weights(w, np.float32(1.0)) == 4
    # the boundary scales with gamma: gamma = 0.25 puts it at 0.125
    assert C.near_boundary_weights(w / 4, np.float32(0.25)) == 4
    assert C.near_boundary_weights(w, np.float32(2.0)) == 0


def test_near_boundary_acts_hand_count():
    """s = 127, so 127x/s = x exactly. Within one fp32 ulp of a half-integer:
    0.5, 1.5, -1.5, 2.5 + ulp(2.5) (4 in row 0). Outside: 2.0, 0.25, 0.5 +
    2^-20. Row 1 (s = 254): x = 1 gives 0.5 (1), x = 3 gives 1.5 (2), x = 2
    gives 1.0 (not)."""
    row0 = np.array([0.5, 1.5, -1.5, 2.5 + 2.0 ** -22, 2.0, 0.25, 0.5 + 2.0 ** -20])
    row1 = np.array([1.0, 3.0, 2.0, 0.0, 0.0, 0.0, 0.0])
    x = np.stack([row0, row1])
    s = np.array([127.0, 254.0])
    assert C.near_boundary_acts(x[:1], s[:1]) == 4
    assert C.near_boundary_acts(x[1:], s[1:]) == 2  # the four zeros give 0.0, not near
    assert C.near_boundary_acts(x, s) == 4 + 2


def test_near_boundary_acts_zero_is_not_a_boundary():
    """0 maps to 0.0, half an integer away from a boundary."""
    assert C.near_boundary_acts(np.zeros((2, 8)), np.array([1.0, 1.0])) == 0


# ---------------------------------------------------------------------------
# sampled-element helpers of the TTQ oracle against its full functions
# ---------------------------------------------------------------------------

def _ttq_case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = O.bf16_round(rng.standard_normal((M, K)))
    w = O.bf16_round(rng.standard_normal((N, K)) * 0.05)
    dY = O.bf16_round(rng.standard_normal((M, N)))
    return O.ttq_layer(x, w, dY), x, dY


@pytest.mark.parametrize("M,N,K", [(5, 7, 9), (6, 6, 6), (3, 11, 4)])
def test_ttq_element_helpers_match_full_functions(M, N, K):
    """ttq_y/dx/dw_elements at every (row, col) equal ttq_forward's y and
    ttq_backward's dX and dW (the same float64 dot products). A square case
    catches an operand taken along the wrong axis."""
    r, x, dY = _ttq_case(M, N, K, 11 + M)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    assert np.allclose(O.ttq_y_elements(x, r["wt"], rows.ravel(), cols.ravel()), r["y"].ravel(), rtol=1e-13,
                       atol=1e-13)
    rows, cols = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    assert np.allclose(O.ttq_dx_elements(dY, r["wt"], rows.ravel(), cols.ravel()), r["dX"].ravel(), rtol=1e-13,
                       atol=1e-13)
    rows, cols = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    assert np.allclose(O.ttq_dw_elements(dY, x, rows.ravel(), cols.ravel()), r["dW"].ravel(), rtol=1e-13,
                       atol=1e-13)


def test_ttq_element_helpers_hand_values():
    """x = [[1, 2]], W_t = [[3, 1], [0, -5]], dY = [[1, -1]]: y = x W_t^T =
    [5, -10], dX = dY W_t = [3, 6], dW = dY^T x = [[1, 2], [-1, -2]]."""
    x = np.array([[1.0, 2.0]])
    wt = np.array([[3.0, 1.0], [0.0, -5.0]])
    dY = np.array([[1.0, -1.0]])
    assert list(O.ttq_y_elements(x, wt, [0, 0], [0, 1])) == [5.0, -10.0]
    assert list(O.ttq_dx_elements(dY, wt, [0, 0], [0, 1])) == [3.0, 6.0]
    assert list(O.ttq_dw_elements(dY, x, [0, 0, 1, 1], [0, 1, 0, 1])) == [1.0, 2.0, -1.0, -2.0]
