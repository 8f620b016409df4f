"""Plain, slow CPU oracle of the TTQ layer (trained ternary quantization).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP library or its Python binding and imports neither.

Source: the web page "TTQ_VERIFICATION.md" (LabStrangeLoop/bitnet), which
summarises Zhu et al., "Trained Ternary Quantization":

* "Algorithm Summary", Forward Pass, Eq. 1: the quantized weight is +Wp where
  W exceeds the threshold delta, -Wn where W is below -delta, 0 elsewhere;
* Initialization (Eq. 2, Section 3.1): delta = 0.7 E|W| and Wp = Wn = E|W|;
* Backward Pass: a straight-through estimator, the latent W receives the
  gradient of the quantized weight unchanged;
* "Bugs Fixed", item 4: pure TTQ, no activation quantization;
* "Bugs Fixed", item 5: the gradient of Wp is the sum of the quantized
  weight's gradient over the positions where the code is positive.

Readings where the page leaves a step open (each is also listed in the design
notes of the repository):

* activations are the layer's bf16 inputs, used unquantized; the products
  run on bf16 operands, so the quantized weight takes the values
  {bf16(Wp), 0, -bf16(Wn)} (round half to even), the way the BitNet path's
  W_hat takes q * bf16(gamma);
* E|W| is the same exactly rounded absmean as the BitNet gamma (fp64 sum,
  rounded to fp32, floored at 1e-8), and delta = fl32(fl32(0.7) * E): one
  fp32 multiplication, as a framework multiplying an fp32 tensor by 0.7 does;
* the threshold test is strict on both sides (Eq. 1), evaluated exactly;
* the gradient of Wn follows from the chain rule on -Wn: minus the sum of
  the quantized weight's gradient over the negative codes (the page writes
  out only the Wp case); delta receives no gradient (the hard threshold has
  derivative zero almost everywhere, and the page gives none);
* the positivity transform (softplus, "Key Design Decisions" item 1) is the
  layer's parametrization: the values here are already positive.
"""

import math

import numpy as np

from . import bitlinear_oracle as B


def ttq_init(w):
    """Initial (delta, Wp, Wn) of a layer with latent weights w
    ("TTQ_VERIFICATION.md", Initialization): E = mean |w| (the absmean of
    the BitNet path, exactly rounded, fp32), delta = fl32(fl32(0.7) * E),
    Wp = Wn = E. Returned as float32 scalars."""
    e = B.absmean_gamma(w)
    delta = np.float32(np.float32(0.7) * np.float32(e))
    return delta, np.float32(e), np.float32(e)


def ttq_codes(w, delta):
    """Eq. 1's selection as codes: +1 where w > delta, -1 where w < -delta,
    0 elsewhere (both comparisons strict, exact: bf16 and fp32 weights and
    the fp32 delta are exact in float64)."""
    w = np.asarray(w, dtype=np.float64)
    d = np.float64(delta)
    return np.where(w > d, 1, np.where(w < -d, -1, 0)).astype(np.int8)


def ttq_values(q, wp, wn):
    """The quantized weight of Eq. 1 as the products use it: bf16(Wp) for
    code +1, -bf16(Wn) for code -1, 0 for code 0 (float64)."""
    q = np.asarray(q)
    p = B.bf16_round(np.float64(wp))
    n = B.bf16_round(np.float64(wn))
    return np.where(q == 1, p, np.where(q == -1, -n, 0.0))


def ttq_forward(x, wt):
    """y = x @ W_t^T in float64 (products of bf16 values are exact)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(wt, dtype=np.float64).T


def ttq_backward(dY, x, q, wp, wn):
    """STE backward ("Backward Pass"; "Bugs Fixed" item 5):
    dX = dY @ W_t, dW = dY^T @ x (the latent weight's gradient equals the
    quantized weight's), grad_Wp = sum of dW over code +1, grad_Wn = minus
    the sum of dW over code -1 (both sums exactly rounded, ``math.fsum``).
    float64 throughout."""
    q = np.asarray(q)
    dY = np.asarray(dY, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    dX = dY @ ttq_values(q, wp, wn)
    dW = dY.T @ x
    g_wp = math.fsum(dW[q == 1].tolist())
    g_wn = -math.fsum(dW[q == -1].tolist())
    return dX, dW, g_wp, g_wn


def ttq_layer(x, w, dY, params=None):
    """The whole TTQ layer on float64 values of the inputs: initial (or
    given) parameters, codes, values, forward and backward."""
    delta, wp, wn = ttq_init(w) if params is None else params
    q = ttq_codes(w, delta)
    wt = ttq_values(q, wp, wn)
    y = ttq_forward(x, wt)
    dX, dW, g_wp, g_wn = ttq_backward(dY, x, q, wp, wn)
    return dict(delta=delta, wp=wp, wn=wn, q=q, wt=wt, y=y, dX=dX, dW=dW, g_wp=g_wp, g_wn=g_wn)


# Single elements, for sampled checks at full size.

def ttq_y_elements(x, wt, rows, cols):
    x = np.asarray(x, dtype=np.float64)
    wt = np.asarray(wt, dtype=np.float64)
    return np.array([float(np.dot(x[m], wt[n])) for m, n in zip(rows, cols)])


def ttq_dx_elements(dY, wt, rows, cols):
    dY = np.asarray(dY, dtype=np.float64)
    wt = np.asarray(wt, dtype=np.float64)
    return np.array([float(np.dot(dY[m], wt[:, k])) for m, k in zip(rows, cols)])


def ttq_dw_elements(dY, x, rows, cols):
    dY = np.asarray(dY, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return np.array([float(np.dot(dY[:, n], x[:, k])) for n, k in zip(rows, cols)])
