"""Parity metrics between a GPU result and the oracle.

TEST INFRASTRUCTURE (see the package docstring). The tolerance rules follow
the forward residual the "bitnet-qat-train" page reports ("Measured
behavior": bf16 output rounding) and the layer's bar of max relative error
<= 8e-3 and normwise error <= 5e-3:

* rel_i = |g_i - o_i| / max(|o_i|, tau). For y, tau = 0: the accumulator is
  exact, so an exact zero must come out as zero (0/0 counts as 0). For dX and
  dW, tau = 2^-8 * RMS(o): an fp32 sum over thousands of terms leaves an
  absolute error around 1e-6..1e-5 of RMS(o), which has no relative bound
  where the exact sum cancels to ~0.
* normwise = ||g - o||_F / ||o||_F.
"""

import numpy as np

MAX_REL = 8e-3
NORMWISE = 5e-3


def rel_errors(got, ref, floor_frac):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    if floor_frac > 0:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
        tau = floor_frac * rms
    else:
        tau = 0.0
    den = np.maximum(np.abs(ref), tau)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(diff == 0, 0.0, diff / den)
    rel = np.where(np.isnan(rel), np.inf, rel)
    nref = float(np.linalg.norm(ref))
    normwise = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got))
    with np.errstate(invalid="ignore", divide="ignore"):
        unfloored = np.where(diff == 0, 0.0, diff / np.abs(ref))
    return dict(
        max_rel=float(np.max(rel)) if rel.size else 0.0,
        normwise=normwise,
        max_rel_unfloored=float(np.nanmax(unfloored)) if unfloored.size else 0.0,
        n_below_floor=int(np.sum(np.abs(ref) < tau)),
        tau=tau,
    )


def check(got, ref, what):
    """Assert the bar for one output: 'y' (no floor) or 'dX'/'dW'/'db',
    'y_bias' and 'y_ttq' (floor 2^-8 RMS: sums in fp32, and a bias or the
    TTQ forward's fp32 sums that can cancel). Returns the metrics."""
    floor = 0.0 if what == "y" else 2.0 ** -8
    m = rel_errors(got, ref, floor)
    assert m["max_rel"] <= MAX_REL, (what, m)
    assert m["normwise"] <= NORMWISE, (what, m)
    return m


def near_boundary_weights(w, gamma):
    """Count of weights within one float32 ulp of the rounding boundary
    |w| = gamma/2 (diagnostic only)."""
    h = np.float32(gamma) * np.float32(0.5)
    ulp = np.spacing(h)
    a = np.abs(np.asarray(w, dtype=np.float64))
    return int(np.sum(np.abs(a - np.float64(h)) <= np.float64(ulp)))


def near_boundary_acts(x, s):
    """Count of activations whose 127*x/s lies within one float32 ulp of a
    half-integer (diagnostic only)."""
    x = np.asarray(x, dtype=np.float64)
    t = 127.0 * x / np.asarray(s, dtype=np.float64)[:, None]
    frac = np.abs(t - np.floor(t) - 0.5)
    ulp = np.spacing(np.abs(t).astype(np.float32)).astype(np.float64)
    return int(np.sum(frac <= ulp))
