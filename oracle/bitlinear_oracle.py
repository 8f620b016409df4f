"""Plain, slow CPU oracle of the BitLinear W1.58/A8 forward and STE backward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP library or its Python binding and imports neither.

Everything is numpy in float64 unless a step fixes another precision. Each
function names the passage it follows. Sources (web pages):

* "1BitTraining.md" (Codys12 gist): ``activation_quant`` and ``weight_quant``
  helpers, the 3-layer net and its identity-STE argument.
* "bitlinear.py" (h4-polytopic-attention): ``ternary_quantize``,
  ``activation_quant_int8`` and ``BitLinear.forward`` (detach-trick STE).
* "bitnet-qat-train" (Hugging Face kernels, phanerozoic): the opening bullets
  (fused ternarize + 2-bit pack, INT8 forward, INT8/2-bit saved state), the
  "Semantics" section (forward formula, INT32 accumulation, STE backward with
  operands rebuilt from saved state, gamma treated as a constant) and
  "Requirements" (bf16 activations, bf16 or f32 master weights).

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):

* epsilon guard: a max-form floor of 1e-8 (fp32) for both gamma and the
  activation scale, so it never perturbs a non-degenerate value;
* gamma: exactly rounded sum of |W| (``math.fsum``), divided by N*K in
  float64, rounded to float32;
* both quantizers are evaluated exactly (round half to even on the exact
  quotient); float64 division followed by ``np.rint`` is exact for these
  operands (argument in ``ternary_codes`` and ``act_quant``);
* the activation scale ``s`` is the per-row absmax (after the floor); 1/127 is
  applied where it is used;
* backward operands: W_hat = q * bf16(gamma), x_hat = bf16(x_q * s / 127)
  (round half to even), both exactly rounded from the exact product;
* the 2-bit format is this project's own (the pages do not give one): row n
  of W is Kp/4 bytes (Kp = K rounded up to a multiple of 64), read as
  little-endian 32-bit words of 16 codes each; the code of W[n, k] sits in
  word k//16 of the row at bit 8*(j%4) + 2*(j//4), j = k%16, as a 2-bit
  two's-complement value (+1 -> 0b01, 0 -> 0b00, -1 -> 0b11); padding codes
  are 0. (Byte b of a word holds the codes j = b, b+4, b+8, b+12.)
"""

import math

import numpy as np

# Floors for the two scales (max form). The pages use 1e-5 ("1BitTraining.md"
# helpers) and 1e-8 ("bitlinear.py"); 1e-8 as a floor is the reading taken.
EPS_W = np.float32(1e-8)
EPS_X = np.float32(1e-8)


# ---------------------------------------------------------------------------
# bf16 helpers (own implementation, float64 arithmetic)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """Value of bf16 bit patterns (uint16) as float64. bf16 is the upper half
    of an IEEE binary32, so every bf16 value is exact in float32 and float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(v):
    """Round float64 values to the nearest bf16 value (8 significant bits),
    ties to even, returned as float64. Only the normal range is needed here
    (the callers' values are >= 1e-8/127 in magnitude or zero); this is
    asserted rather than handled."""
    v = np.asarray(v, dtype=np.float64)
    nz = v != 0
    if np.any(np.abs(v[nz]) < 2.0 ** -126):
        raise ValueError("bf16_round: subnormal result not supported by the oracle")
    m, e = np.frexp(v)                  # v = m * 2**e with 0.5 <= |m| < 1
    r = np.rint(np.ldexp(m, 8))         # 8 significant bits, half to even
    out = np.ldexp(r, e - 8)
    if not np.all(np.isfinite(out)):
        raise ValueError("bf16_round: overflow")
    return out


# ---------------------------------------------------------------------------
# Weights: absmean scale, RoundClip ternarization, 2-bit packing
# ---------------------------------------------------------------------------

def absmean_gamma(w):
    """Per-tensor absmean scale gamma = mean(|W|).

    Follows "1BitTraining.md" (``weight_quant``: scale from the mean of |w|),
    "bitlinear.py" (``ternary_quantize``: ``scale = mean(|w|)``) and
    "bitnet-qat-train" (opening paragraph: per-tensor absmean weight scale).
    The sum is exactly rounded to float64 (``math.fsum``), divided by the
    element count in float64, rounded to float32 and floored at EPS_W.
    """
    a = np.abs(np.asarray(w, dtype=np.float64)).ravel()
    if a.size == 0:
        raise ValueError("absmean_gamma: empty tensor")
    mean = math.fsum(a) / a.size
    g = np.float32(mean)
    return np.float32(max(g, EPS_W))


def ternary_codes(w, gamma):
    """RoundClip(W / gamma, -1, +1): round half to even, then clip.

    Follows "bitlinear.py" ``ternary_quantize`` (round of w/scale, clamp to
    [-1, 1]) and "1BitTraining.md" ``weight_quant`` (round, clip to +-1).

    Exactness of the float64 evaluation: with W = a*2^p and gamma = b*2^r
    (a, b integers < 2^24), a quotient Q in [1/4, 2] that is not exactly a
    half-integer h in {0.5, 1.5} satisfies |Q - h| > 2^-27, while float64
    division errs by at most 2^-52 there; exact half-integers are
    representable and returned exactly. So rint(fl64(Q)) = RNE(Q).
    """
    q = np.rint(np.asarray(w, dtype=np.float64) / np.float64(gamma))
    return np.clip(q, -1, 1).astype(np.int8)


def k_pad(K):
    """Padded reduction length Kp: K rounded up to a multiple of 64."""
    return ((int(K) + 63) // 64) * 64


def code_bit(j):
    """Bit offset of code j (0..15) inside its 32-bit word."""
    return 8 * (j % 4) + 2 * (j // 4)


def pack_codes(q, Kp=None):
    """2-bit packing of ternary codes [N, K] into bytes [N, Kp/4].

    The pages state that the fused pass packs 2 bits per weight
    ("bitnet-qat-train", opening bullets) but give no format; the format here
    is this project's: 16 codes per little-endian 32-bit word, code j of word
    w (k = 16w + j) at bit 8*(j%4) + 2*(j//4), two's complement (+1 -> 01,
    0 -> 00, -1 -> 11), zero codes in the padding.
    """
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    if Kp is None:
        Kp = k_pad(K)
    full = np.zeros((N, Kp), dtype=np.int64)
    full[:, :K] = q
    f = (full & 3).reshape(N, Kp // 16, 16)
    words = np.zeros((N, Kp // 16), dtype=np.int64)
    for j in range(16):
        words |= f[..., j] << code_bit(j)
    return words.astype("<u4").view(np.uint8).reshape(N, Kp // 4)


def unpack_codes(packed, K):
    """Inverse of ``pack_codes``: bytes [N, Kp/4] -> codes int8 [N, K].
    The unused field value 0b10 raises."""
    p = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    N = p.shape[0]
    words = p.view("<u4").astype(np.int64)
    fields = np.stack([(words >> code_bit(j)) & 3 for j in range(16)], axis=-1)
    if np.any(fields == 2):
        raise ValueError("unpack_codes: field value 0b10 is never written")
    vals = np.where(fields == 3, -1, fields).reshape(N, -1)
    return vals[:, :K].astype(np.int8)


# ---------------------------------------------------------------------------
# Activations: per-token absmax int8
# ---------------------------------------------------------------------------

def act_quant(x, Kp=None):
    """Per-token absmax int8 quantization.

    Follows "bitlinear.py" ``activation_quant_int8`` (scale = row absmax with
    a floor; x_q = clamp(round(x*127/scale), -127, 127)) and
    "1BitTraining.md" ``activation_quant`` (127/absmax, round, clip; its
    clip at -128 is never reached since |x*127/s| <= 127).

    Returns (x_q int8 [M, Kp] with zero padding, s float32 [M]) where s is
    the floored absmax (exact in float32 for bf16 inputs).

    Exactness of the float64 evaluation: 127*x is exact; writing 127*x =
    a*2^p, s = b*2^r (a < 2^31, b < 2^24), a quotient >= 1/2 that is not a
    half-integer lies more than 2^-33 from every half-integer, far above the
    float64 division error (<= 2^-46 for quotients <= 127), and exact
    half-integers come out exactly. So rint(fl64(127*x/s)) = RNE(127*x/s).
    """
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if Kp is None:
        Kp = k_pad(K)
    if K > 0:
        amax = np.max(np.abs(x), axis=1)
    else:
        amax = np.zeros(M)
    amax32 = amax.astype(np.float32)
    if not np.array_equal(amax32.astype(np.float64), amax):
        raise ValueError("act_quant: inputs must be float32-representable")
    s = np.maximum(amax32, EPS_X)
    q = np.rint((127.0 * x) / s.astype(np.float64)[:, None])
    q = np.clip(q, -127, 127)
    xq = np.zeros((M, Kp), dtype=np.int8)
    xq[:, :K] = q.astype(np.int8)
    return xq, s


# ---------------------------------------------------------------------------
# Forward: INT32 accumulation, rescale
# ---------------------------------------------------------------------------

def forward_acc(x_q, q):
    """acc[m, n] = sum_k x_q[m, k] * q[n, k], exact ("bitnet-qat-train",
    Semantics: INT32 accumulation). Computed with a float64 matmul, which is
    exact here because every partial sum is an integer of magnitude
    <= 127*K < 2^53; the bound 127*K < 2^31 is asserted."""
    q = np.asarray(q)
    K = q.shape[1]
    if 127 * K >= 2 ** 31:
        raise ValueError("forward_acc: 127*K must stay below 2^31")
    a = np.asarray(x_q)[:, :K].astype(np.float64) @ q.astype(np.float64).T
    return a.astype(np.int64)


def forward_y(acc, s, gamma):
    """y = acc * (s/127) * gamma in float64, unrounded: the comparison target
    for the bf16 output ("bitnet-qat-train", Semantics: quant(x) times
    ternarize(W)^T, scaled by the activation scale and gamma)."""
    s64 = np.asarray(s, dtype=np.float64)[:, None]
    return np.asarray(acc, dtype=np.float64) * (s64 / 127.0) * np.float64(gamma)


# ---------------------------------------------------------------------------
# STE backward with operands rebuilt from the saved state
# ---------------------------------------------------------------------------

def w_hat(q, gamma):
    """W_hat = q * bf16(gamma): the ternary weight dequantized in bf16
    ("bitnet-qat-train", Semantics: W_hat rebuilt from the 2-bit state)."""
    g16 = bf16_round(np.float64(gamma))
    return np.asarray(q, dtype=np.float64) * g16


def x_hat(x_q, s, K):
    """x_hat = bf16(x_q * s / 127), round half to even on the exact value
    ("bitnet-qat-train", Semantics: x_hat rebuilt from the INT8 state).
    x_q*s is exact in float64 and the division rounds once; the bf16
    rounding of that float64 equals the rounding of the exact quotient
    (a bf16 midpoint can only be hit exactly, never missed by 2^-53)."""
    xq = np.asarray(x_q)[:, :K].astype(np.float64)
    s64 = np.asarray(s, dtype=np.float64)[:, None]
    return bf16_round(xq * s64 / 127.0)


def backward(dY, x_q, s, q, gamma):
    """Straight-through estimator backward ("bitnet-qat-train", Semantics;
    "bitlinear.py" ``BitLinear.forward`` detach trick; "1BitTraining.md",
    identity-STE): dX = dY @ W_hat and dW = dY^T @ x_hat, gamma treated as a
    constant. float64; products of bf16 values are exact in float64."""
    q = np.asarray(q)
    K = q.shape[1]
    dY = np.asarray(dY, dtype=np.float64)
    dX = dY @ w_hat(q, gamma)
    dW = dY.T @ x_hat(x_q, s, K)
    return dX, dW


def layer_fwd_bwd(x, w, dY, with_backward=True):
    """The whole layer on float64 values of the inputs (bf16 x and dY, bf16
    or f32 W): ternarize + pack, act-quant, forward, STE backward."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    Kp = k_pad(K)
    gamma = absmean_gamma(w)
    q = ternary_codes(w, gamma)
    packed = pack_codes(q, Kp)
    x_q, s = act_quant(x, Kp)
    acc = forward_acc(x_q, q)
    y = forward_y(acc, s, gamma)
    out = dict(gamma=gamma, q=q, packed=packed, x_q=x_q, s=s, acc=acc, y=y)
    if with_backward:
        dX, dW = backward(dY, x_q, s, q, gamma)
        out.update(dX=dX, dW=dW)
    return out


# ---------------------------------------------------------------------------
# Bias
# ---------------------------------------------------------------------------

def forward_y_bias(acc, s, gamma, bias):
    """y + bias[n]: the optional bias of "bitlinear.py" (BitLinear.forward,
    added after the product), on bf16 bias values; float64."""
    return forward_y(acc, s, gamma) + np.asarray(bias, dtype=np.float64)[None, :]


def bias_grad(dY):
    """db[n] = sum over tokens of dY[m, n], the gradient of that bias,
    exactly rounded (``math.fsum`` per column)."""
    d = np.asarray(dY, dtype=np.float64)
    return np.array([math.fsum(d[:, n]) for n in range(d.shape[1])])


# ---------------------------------------------------------------------------
# 1-bit sign gradients
# ---------------------------------------------------------------------------

def sign1_pack(dW, Kp=None):
    """1-bit signs of the weight gradient dW [N, K], packed into bytes
    [N, Kp/8], for a sign-based optimiser ("1BitTraining.md", the closing
    paragraphs: the identity-STE gradient has the sign of the gradient with
    respect to the quantised weight, so a device holding only the 2-bit
    weights can stream 1-bit gradients). The page's check uses a
    three-valued sign; with one bit, zero goes with the non-negative side
    (the reading taken): the bit of dW[n, k] is 1 iff dW[n, k] < 0. Bit j of
    byte b of row n holds k = 8b + j; columns k >= K are 0."""
    d = np.asarray(dW, dtype=np.float64)
    N, K = d.shape
    if Kp is None:
        Kp = k_pad(K)
    neg = np.zeros((N, Kp), dtype=np.int64)
    neg[:, :K] = d < 0
    bits = neg.reshape(N, Kp // 8, 8)
    out = np.zeros((N, Kp // 8), dtype=np.int64)
    for j in range(8):
        out |= bits[..., j] << j
    return out.astype(np.uint8)


def sign1_unpack(packed, K):
    """Inverse of ``sign1_pack`` up to zeros: bytes [N, Kp/8] -> int8 [N, K]
    with -1 where the bit is set and +1 elsewhere."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    N = p.shape[0]
    bits = np.stack([(p >> j) & 1 for j in range(8)], axis=-1).reshape(N, -1)[:, :K]
    return np.where(bits == 1, -1, 1).astype(np.int8)


# ---------------------------------------------------------------------------
# Single elements, for sampled checks at full size
# ---------------------------------------------------------------------------

def acc_elements(x_q, q, rows, cols):
    """acc at the (rows[i], cols[i]) pairs, exact int64."""
    q = np.asarray(q)
    K = q.shape[1]
    a = np.asarray(x_q)[rows, :K].astype(np.int64)
    b = q[cols, :].astype(np.int64)
    return np.sum(a * b, axis=1)


def y_elements(x_q, s, q, gamma, rows, cols):
    acc = acc_elements(x_q, q, rows, cols).astype(np.float64)
    return acc * (np.asarray(s, np.float64)[rows] / 127.0) * np.float64(gamma)


def dx_elements(dY, q, gamma, rows, cols):
    """dX[m, k] = sum_n dY[m, n] * W_hat[n, k] at (rows=m, cols=k) pairs."""
    dY = np.asarray(dY)
    g16 = bf16_round(np.float64(gamma))
    a = dY[rows, :].astype(np.float64)
    b = np.asarray(q)[:, cols].T.astype(np.float64) * g16
    return np.sum(a * b, axis=1)


def dw_elements(dY, x_q, s, rows, cols):
    """dW[n, k] = sum_m dY[m, n] * x_hat[m, k] at (rows=n, cols=k) pairs."""
    dY = np.asarray(dY)
    a = dY[:, rows].T.astype(np.float64)
    xq = np.asarray(x_q)[:, cols].T.astype(np.float64)
    xh = bf16_round(xq * np.asarray(s, np.float64)[None, :] / 127.0)
    return np.sum(a * xh, axis=1)
