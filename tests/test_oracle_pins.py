"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: exact
rational arithmetic (``fractions.Fraction``, Python ints), closed forms,
invariants, statistics of the input distributions, an independent autograd
route, and the values the pages print. No GPU.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from ternary_weight_quantization_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# exact helpers (Fraction based, independent of the oracle)
# ---------------------------------------------------------------------------

def rne_int(fr):
    """Round a Fraction to the nearest integer, ties to even."""
    fl = math.floor(fr)
    d = fr - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def rne_bf16(fr):
    """Round a nonzero Fraction to 8 significant bits, ties to even."""
    if fr == 0:
        return Fraction(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 256:
        a /= 2
        e += 1
    while a < 128:
        a *= 2
        e -= 1
    r = rne_int(a)
    return sgn * Fraction(r) * (Fraction(2) ** e)


def bf16_vals(rng, shape, scale=1.0):
    return WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(
        (rng.standard_normal(shape) * scale).astype(np.float32))).astype(np.float64)


# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------

def test_bf16_round_matches_exact_rounding():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))
    # add exact midpoints between neighbouring bf16 values (tie cases)
    mids = (np.arange(128, 256, dtype=np.float64) + 0.5) * 2.0 ** -7
    v = np.concatenate([v, mids, -mids * 4])
    got = O.bf16_round(v)
    for a, g in zip(v, got):
        assert Fraction(g) == rne_bf16(Fraction(a))


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(v) & (v != 0) & (np.abs(v) >= 2.0 ** -126)
    # every finite normal bf16 value is a fixed point of bf16 rounding
    assert np.array_equal(O.bf16_round(v[fin]), v[fin])
    # and agrees with the input generator's decoding
    assert np.array_equal(WL.bf16_bits_to_f32(bits)[fin].astype(np.float64), v[fin])


# ---------------------------------------------------------------------------
# gamma
# ---------------------------------------------------------------------------

def test_gamma_closed_forms():
    assert O.absmean_gamma(np.full((3, 5), -0.375)) == np.float32(0.375)
    assert O.absmean_gamma(np.array([[2.0, 0.5, 1.0, 0.5]])) == np.float32(1.0)
    # mean of |U(-a, a)| = a/2 (1M samples: within 0.3 %)
    rng = np.random.default_rng(2)
    w = rng.uniform(-0.2, 0.2, (1000, 1000))
    assert abs(O.absmean_gamma(w) - 0.1) < 3e-4
    # all-zero tensor: the floor
    assert O.absmean_gamma(np.zeros((4, 4))) == np.float32(1e-8)


def test_gamma_float32_rounding_ties_to_even():
    u = 2.0 ** -23
    # mean = 1 + 2^-24: halfway between 1 and 1 + 2^-23 -> even (1)
    assert O.absmean_gamma(np.array([1.0, 1.0 + u])) == np.float32(1.0)
    # mean = 1 + 1.5 * 2^-23: halfway between 1+u (odd) and 1+2u (even)
    assert O.absmean_gamma(np.array([1.0 + u, 1.0 + 2 * u])) == np.float32(1.0 + 2 * u)


def test_gamma_exact_sum_vs_fraction():
    rng = np.random.default_rng(3)
    for trial in range(20):
        n = int(rng.integers(1, 300))
        w = (rng.standard_normal(n) * np.exp(rng.uniform(-30, 30, n))).astype(np.float32)
        if trial == 0:
            w = np.array([1e30, 1.0, -1e30, 1e-30, 3.0], dtype=np.float32)
            n = w.size
        s = sum(Fraction(float(a)) for a in np.abs(w.astype(np.float64)))
        mean = float(s) / n  # float(Fraction) and float / int round correctly
        want = max(np.float32(mean), np.float32(1e-8))
        assert O.absmean_gamma(w) == want


# ---------------------------------------------------------------------------
# ternary codes
# ---------------------------------------------------------------------------

def test_codes_hand_examples_and_ties():
    # gamma = 1; 0.5 is a tie (-> 0), 1.5 rounds to 2 and clips to 1
    w = np.array([[2.0, 0.5, 1.0, 0.5]])
    g = O.absmean_gamma(w)
    assert g == 1.0
    assert O.ternary_codes(w, g).tolist() == [[1, 0, 1, 0]]
    w = np.array([[1.5, -0.5, -1.0, 1.0]])
    g = O.absmean_gamma(w)
    assert g == 1.0
    assert O.ternary_codes(w, g).tolist() == [[1, 0, -1, 1]]
    w = np.array([[-3.0, 0.25, -0.5, 0.25]])
    g = O.absmean_gamma(w)
    assert g == 1.0
    assert O.ternary_codes(w, g).tolist() == [[-1, 0, 0, 0]]


def test_codes_constant_tensor():
    for c in (0.7, -0.02, 3.0):
        w = np.full((5, 9), c, dtype=np.float32)
        g = O.absmean_gamma(w)
        assert np.all(O.ternary_codes(w, g) == np.sign(c))


def test_codes_vs_fraction_bruteforce():
    rng = np.random.default_rng(4)
    for dt in ("f32", "bf16"):
        w = rng.standard_normal((12, 40)).astype(np.float32) * np.float32(0.05)
        if dt == "bf16":
            w = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(w))
        g = O.absmean_gamma(w)
        h = np.float32(g) * np.float32(0.5)
        # plant exact ties and their float32 neighbours
        w[0, :6] = [h, -h, np.nextafter(h, np.float32(1)), np.nextafter(h, np.float32(0)),
                    np.float32(3) * h, -np.float32(3) * h]
        g = O.absmean_gamma(w)
        q = O.ternary_codes(w, g)
        G = Fraction(float(g))
        for a, c in zip(w.astype(np.float64).ravel(), q.ravel()):
            want = max(-1, min(1, rne_int(Fraction(float(a)) / G)))
            assert want == c
        assert set(np.unique(q)).issubset({-1, 0, 1})


def test_codes_zero_fraction_statistics():
    """Closed forms for the share of zero codes, which pin both gamma (mean of
    |W|) and the rounding threshold (gamma / 2)."""
    rng = np.random.default_rng(5)
    # U(-a, a): gamma = a/2, zero iff |w| <= a/4 -> probability 1/4
    w = rng.uniform(-1, 1, 2_000_000)
    q = O.ternary_codes(w, O.absmean_gamma(w))
    assert abs(np.mean(q == 0) - 0.25) < 2e-3
    # N(0, 1): gamma = sqrt(2/pi), zero iff |z| <= gamma/2
    z = rng.standard_normal(2_000_000)
    q = O.ternary_codes(z, O.absmean_gamma(z))
    p = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    assert abs(np.mean(q == 0) - p) < 2e-3 and abs(p - 0.3101) < 1e-3
    # 10 % exact zeros + N(0, s): gamma = 0.9 s sqrt(2/pi)
    z = rng.standard_normal(2_000_000) * 0.02
    z[rng.choice(z.size, z.size // 10, replace=False)] = 0.0
    q = O.ternary_codes(z, O.absmean_gamma(z))
    p = 0.1 + 0.9 * math.erf(0.9 * math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    assert abs(np.mean(q == 0) - p) < 2e-3 and abs(p - 0.3524) < 1e-3


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------

def test_pack_hand_bytes():
    # codes of k = 0..3 are the lowest field of bytes 0..3 of the first word:
    # +1, 0, -1, +1 -> 0x01, 0x00, 0x03, 0x01
    q = np.array([[1, 0, -1, 1]], dtype=np.int8)
    p = O.pack_codes(q, 64)
    assert p.shape == (1, 16)
    assert p[0, :4].tolist() == [0x01, 0x00, 0x03, 0x01]
    assert np.all(p[0, 4:] == 0)
    # k = 4..7 go to bits 2..3 of bytes 0..3, k = 8..11 to bits 4..5, k = 12..15
    # to bits 6..7
    q = np.array([[-1, -1, -1, -1, 1, 1, 1, 1, 0, 0, 0, -1, 1, 0, 0, 0]], dtype=np.int8)
    p = O.pack_codes(q)
    assert p[0, :4].tolist() == [0b01_00_01_11, 0b00_00_01_11, 0b00_00_01_11, 0b00_11_01_11]
    # word w holds k = 16w..16w+15; code j of the word at bit 8*(j%4) + 2*(j//4)
    q = np.zeros((1, 64), dtype=np.int8)
    q[0, 17] = -1   # word 1, j = 1 -> bit 8
    q[0, 30] = 1    # word 1, j = 14 -> bit 16 + 6 = 22
    word = O.pack_codes(q).view("<u4")[0, 1]
    assert word == (3 << 8) | (1 << 22)
    # byte b of a word holds codes j = b, b+4, b+8, b+12 (the planar property
    # used to expand 4 codes with one shift and one mask)
    for t in range(4):
        q = np.zeros((1, 16), dtype=np.int8)
        q[0, 4 * t:4 * t + 4] = [1, -1, 1, -1]
        w = int(O.pack_codes(q).view("<u4")[0, 0])
        assert (w >> (2 * t)) & 0x03030303 == 0x03010301


def test_pack_roundtrip_and_padding():
    rng = np.random.default_rng(6)
    for K in (1, 7, 63, 64, 65, 200):
        q = rng.integers(-1, 2, size=(9, K)).astype(np.int8)
        p = O.pack_codes(q)
        assert p.shape == (9, O.k_pad(K) // 4)
        assert np.array_equal(O.unpack_codes(p, K), q)
        tail = O.unpack_codes(p, O.k_pad(K))[:, K:]
        assert np.all(tail == 0)


# ---------------------------------------------------------------------------
# activation quantization
# ---------------------------------------------------------------------------

def test_act_quant_invariants():
    rng = np.random.default_rng(7)
    x = bf16_vals(rng, (64, 300))
    xq, s = O.act_quant(x)
    assert xq.shape == (64, O.k_pad(300))
    assert np.all(xq[:, 300:] == 0)
    assert np.all(np.abs(xq.astype(int)) <= 127)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(xq[np.arange(64), am].astype(int)) == 127)
    err = np.abs(x - xq[:, :300] * s[:, None].astype(np.float64) / 127.0)
    s64 = s[:, None].astype(np.float64)
    assert np.all(err <= s64 / 254.0 + 1e-13 * s64)
    assert np.array_equal(s.astype(np.float64), np.max(np.abs(x), axis=1))


def test_act_quant_vs_fraction_and_ties():
    rng = np.random.default_rng(8)
    x = bf16_vals(rng, (6, 50))
    # row 1: absmax with significand 254/128, elements (2j+1)/128 give
    # 127x/s = j + 1/2 exactly
    s_t = 254.0 / 128.0
    x[1, :] = 0
    x[1, 0] = s_t
    for j in range(1, 40):
        x[1, j] = (2 * j + 1) / 128.0 * (1 if j % 3 else -1)
    # row 2: x = s/2 gives 63.5 -> 64
    x[2, :] = 0
    x[2, 0] = -3.0
    x[2, 1] = 1.5
    # row 3: all zero
    x[3, :] = 0
    xq, s = O.act_quant(x)
    assert s[3] == np.float32(1e-8) and np.all(xq[3] == 0)
    assert xq[2, 1] == 64 and xq[2, 0] == -127
    for j in range(1, 40):
        want = rne_int(Fraction(2 * j + 1, 2))
        assert abs(int(xq[1, j])) == want
        assert want % 2 == 0
    for m in range(6):
        S = Fraction(float(s[m]))
        for k in range(50):
            want = max(-127, min(127, rne_int(127 * Fraction(float(x[m, k])) / S)))
            assert int(xq[m, k]) == want


def test_act_quant_exhaustive_bf16_significands():
    """Every bf16 significand of the scale s in [1, 2) against every bf16 x
    with s/256 < x <= s (smaller x round to 0 trivially), checked against
    exact integer round-half-even of 127*x/s."""
    sig = np.arange(128, 256, dtype=np.int64)          # 8-bit significands
    S = np.repeat(sig, 128 * 9)                       # s = S / 128
    X = np.tile(np.tile(sig, 9), 128)                 # x = X / 128 * 2^-d
    D = np.tile(np.repeat(np.arange(9), 128), 128)
    keep = (X * 2.0 ** -D) <= S
    S, X, D = S[keep], X[keep], D[keep]
    num = 127 * X
    den = S << D
    q = num // den
    r = num - q * den
    up = (2 * r > den) | ((2 * r == den) & (q % 2 == 1))
    want = q + up
    s_val = S / 128.0
    x_val = X / 128.0 * 2.0 ** -D
    rows = np.stack([s_val, x_val], axis=1)
    xq, s = O.act_quant(rows)
    assert np.array_equal(s.astype(np.float64), s_val)
    assert np.array_equal(xq[:, 1].astype(np.int64), want)
    assert len(want) > 100_000


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def test_forward_acc_bruteforce_python_ints():
    rng = np.random.default_rng(9)
    for (M, K, N) in [(3, 5, 4), (2, 7, 6), (5, 70, 3)]:
        x = bf16_vals(rng, (M, K))
        w = rng.uniform(-1, 1, (N, K)).astype(np.float32)
        g = O.absmean_gamma(w)
        q = O.ternary_codes(w, g)
        xq, s = O.act_quant(x)
        acc = O.forward_acc(xq, q)
        for m in range(M):
            for n in range(N):
                want = sum(int(xq[m, k]) * int(q[n, k]) for k in range(K))
                assert acc[m, n] == want
        # padding columns take no part
        xq2 = xq.copy()
        xq2[:, K:] = 99
        assert np.array_equal(O.forward_acc(xq2, q), acc)
        rows = rng.integers(0, M, 10)
        cols = rng.integers(0, N, 10)
        assert np.array_equal(O.acc_elements(xq, q, rows, cols), acc[rows, cols])


def test_y_dx_dw_exact_fractions():
    rng = np.random.default_rng(10)
    M, K, N = 3, 6, 5
    x = bf16_vals(rng, (M, K))
    w = rng.uniform(-0.3, 0.3, (N, K)).astype(np.float32)
    dY = bf16_vals(rng, (M, N))
    r = O.layer_fwd_bwd(x, w, dY)
    g = Fraction(float(r["gamma"]))
    g16 = rne_bf16(g)
    xq, s, q = r["x_q"], r["s"], r["q"]
    xh = [[rne_bf16(int(xq[m, k]) * Fraction(float(s[m])) / 127) for k in range(K)]
          for m in range(M)]
    for m in range(M):
        for n in range(N):
            acc = sum(int(xq[m, k]) * int(q[n, k]) for k in range(K))
            want = acc * Fraction(float(s[m])) / 127 * g
            assert abs(Fraction(r["y"][m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)
        for k in range(K):
            want = sum(Fraction(float(dY[m, n])) * int(q[n, k]) * g16 for n in range(N))
            assert abs(Fraction(r["dX"][m, k]) - want) <= Fraction(1, 2 ** 48)
    for n in range(N):
        for k in range(K):
            want = sum(Fraction(float(dY[m, n])) * xh[m][k] for m in range(M))
            assert abs(Fraction(r["dW"][n, k]) - want) <= Fraction(1, 2 ** 48)
    rows = np.array([0, 2, 1])
    cols = np.array([3, 0, 4])
    assert np.allclose(O.y_elements(xq, s, q, r["gamma"], rows, cols), r["y"][rows, cols], rtol=1e-15)
    assert np.allclose(O.dx_elements(dY, q, r["gamma"], rows, cols), r["dX"][rows, cols], rtol=1e-14)
    rows_n = np.array([4, 0, 2])
    assert np.allclose(O.dw_elements(dY, xq, s, rows_n, cols), r["dW"][rows_n, cols], rtol=1e-14)


def test_forward_constant_weight_closed_form():
    rng = np.random.default_rng(11)
    x = bf16_vals(rng, (4, 33))
    c = 0.25
    w = np.full((7, 33), -c)
    r = O.layer_fwd_bwd(x, w, np.zeros((4, 7)))
    row = -np.sum(r["x_q"][:, :33].astype(np.float64), axis=1) * r["s"] / 127.0 * c
    assert np.allclose(r["y"], np.repeat(row[:, None], 7, axis=1), rtol=1e-15, atol=0)


def test_backward_one_hot_dY_selects_rows():
    """dY with a single 1 at (m0, n0): dX[m0] = W_hat[n0], dW[n0] = x_hat[m0],
    all else 0. Catches swapped or transposed operands."""
    rng = np.random.default_rng(12)
    M, K, N = 5, 9, 7
    x = bf16_vals(rng, (M, K))
    w = rng.uniform(-0.3, 0.3, (N, K))
    dY = np.zeros((M, N))
    m0, n0 = 3, 5
    dY[m0, n0] = 1.0
    r = O.layer_fwd_bwd(x, w, dY)
    wh = O.w_hat(r["q"], r["gamma"])
    xh = O.x_hat(r["x_q"], r["s"], K)
    assert np.array_equal(r["dX"][m0], wh[n0])
    assert np.all(np.delete(r["dX"], m0, axis=0) == 0)
    assert np.array_equal(r["dW"][n0], xh[m0])
    assert np.all(np.delete(r["dW"], n0, axis=0) == 0)
    # W_hat entries are exactly +-bf16(gamma) or 0
    g16 = float(rne_bf16(Fraction(float(r["gamma"]))))
    assert set(np.unique(np.abs(wh))).issubset({0.0, g16})


def test_against_torch_autograd_detach_ste():
    """Independent route: the detach-trick STE module of "bitlinear.py"
    (BitLinear.forward) in torch float64 on the CPU, fed with the same
    dequantized operands, gives the oracle's y, dX and dW."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    M, K, N = 16, 40, 24
    x = bf16_vals(rng, (M, K))
    w = rng.uniform(-1 / math.sqrt(K), 1 / math.sqrt(K), (N, K)).astype(np.float32)
    dY = bf16_vals(rng, (M, N))
    r = O.layer_fwd_bwd(x, w, dY)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w.astype(np.float64), requires_grad=True)
    x_fq = torch.tensor(r["x_q"][:, :K].astype(np.float64) * r["s"][:, None].astype(np.float64) / 127.0)
    # forward with gamma (fp32), as in the INT8 forward
    w_fq = torch.tensor(r["q"].astype(np.float64) * float(r["gamma"]))
    y = torch.nn.functional.linear(xt + (x_fq - xt).detach(), wt + (w_fq - wt).detach())
    assert np.allclose(y.detach().numpy(), r["y"], rtol=1e-12, atol=1e-12 * np.abs(r["y"]).max())
    # backward with the rebuilt operands (x_hat, W_hat)
    xh = torch.tensor(O.x_hat(r["x_q"], r["s"], K))
    wh = torch.tensor(O.w_hat(r["q"], r["gamma"]))
    y2 = torch.nn.functional.linear(xt + (xh - xt).detach(), wt + (wh - wt).detach())
    y2.backward(torch.tensor(dY))
    assert np.allclose(xt.grad.numpy(), r["dX"], rtol=1e-12, atol=1e-12)
    assert np.allclose(wt.grad.numpy(), r["dW"], rtol=1e-12, atol=1e-12)


def test_bias_against_torch_autograd():
    """The optional bias of "bitlinear.py" (BitLinear.forward: F.linear of
    the STE operands with self.bias) in torch float64: its output and the
    bias gradient torch's autograd gives equal the oracle's forward_y_bias
    and bias_grad."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    M, K, N = 12, 72, 20
    x = bf16_vals(rng, (M, K))
    w = rng.uniform(-1 / math.sqrt(K), 1 / math.sqrt(K), (N, K)).astype(np.float32)
    b = bf16_vals(rng, (N,), 0.1)
    dY = bf16_vals(rng, (M, N))
    r = O.layer_fwd_bwd(x, w, dY, with_backward=False)
    xt = torch.tensor(x)
    bt = torch.tensor(b, requires_grad=True)
    x_fq = torch.tensor(r["x_q"][:, :K].astype(np.float64) * r["s"][:, None].astype(np.float64) / 127.0)
    w_fq = torch.tensor(r["q"].astype(np.float64) * float(r["gamma"]))
    y = torch.nn.functional.linear(xt + (x_fq - xt).detach(), w_fq, bt)
    ref = O.forward_y_bias(r["acc"], r["s"], r["gamma"], b)
    assert np.allclose(y.detach().numpy(), ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    y.backward(torch.tensor(dY))
    assert np.allclose(bt.grad.numpy(), O.bias_grad(dY), rtol=1e-12, atol=1e-12)


def test_bias_grad_exact_column_sums():
    """bias_grad against exact Fraction column sums (3 x 5 and a ragged
    7 x 1), which a row sum or a transposed operand would not give."""
    rng = np.random.default_rng(19)
    for M, N in ((3, 5), (7, 1), (64, 9)):
        d = bf16_vals(rng, (M, N))
        exact = [float(sum(Fraction(float(d[m, n])) for m in range(M))) for n in range(N)]
        assert np.array_equal(O.bias_grad(d), np.array(exact)), (M, N)
    assert np.array_equal(O.bias_grad(np.array([[1.0, 2.0, 3.0], [10.0, 20.0, 30.0]])), [11.0, 22.0, 33.0])


# ---------------------------------------------------------------------------
# the tiny 3-layer net of "1BitTraining.md"
# ---------------------------------------------------------------------------

def _golden_signs():
    out = {}
    for line in open(os.path.join(GOLDEN, "tiny_net_sign_equality.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = v == "True"
    return out


def _fake_quant(torch, v, scale, lo, hi):
    """v on the integer grid of `scale`: round half to even, clip to
    [lo, hi], divide back (the quantizers of "1BitTraining.md", opening
    helpers, stated as formulas: activations scale each row so its absmax
    maps to 127, weights scale by the reciprocal mean of |W|, each scale
    floored at 1e-5; activations clip to [-128, 127], weights to [-1, 1])."""
    return torch.clamp(torch.round(v * scale), lo, hi) / scale


def test_tiny_net_page_result_reproduces():
    """The page's own net ("1BitTraining.md", Multilayer check: 7 -> 6 -> 5 ->
    4, batch 2, float64, every hidden output fake-quantized, the last not,
    squared-error loss against a random target), with the gradients taken by
    torch autograd rather than by hand: the STE gradient of each latent
    weight has the sign of the gradient of the quantised weight, element by
    element, as printed on the page."""
    torch = pytest.importorskip("torch")
    d = WL.tiny_net_inputs()
    floor, act_range, w_range = 1e-5, (-128, 127), (-1, 1)

    def act_fq(v):
        return _fake_quant(torch, v, 127.0 / torch.clamp(v.abs().amax(dim=-1, keepdim=True), min=floor), *act_range)

    def weight_fq(w):
        return _fake_quant(torch, w, 1.0 / torch.clamp(w.abs().mean(), min=floor), *w_range)

    def through(v, fq):  # identity straight-through estimator: value fq, gradient of v
        return v + (fq - v).detach()

    def loss_of(weights):
        act = act_fq(torch.tensor(d["x0"]))
        for depth, w in enumerate(weights):
            pre = act @ w.T
            act = pre if depth == len(weights) - 1 else through(pre, act_fq(pre))
        return 0.5 * ((act - torch.tensor(d["target"])) ** 2).sum()

    latent = [torch.tensor(w, requires_grad=True) for w in d["Ws"]]
    quantised = [weight_fq(w.detach()).clone().requires_grad_(True) for w in latent]
    loss_of(quantised).backward()
    loss_of([through(w, weight_fq(w)) for w in latent]).backward()
    golden = _golden_signs()
    for i, (w, q) in enumerate(zip(latent, quantised)):
        same = bool(torch.all(torch.sign(w.grad) == torch.sign(q.grad)))
        assert same == golden[f"layer{i + 1}"]
        assert float(q.grad.abs().min()) > 0.1


def test_tiny_net_oracle_ste_signs():
    """The same net through the oracle's layer functions at the ABI's
    precisions (bf16 activations, float32 master weights, bf16 layer outputs):
    sign(STE dW_i) equals sign(dL/dQ_i) from torch autograd with
    Q_i = q_i * bf16(gamma_i) as leaves, for every element."""
    torch = pytest.importorskip("torch")
    d = WL.tiny_net_inputs()
    Ws = [w.astype(np.float32) for w in d["Ws"]]
    x = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(d["x0"].astype(np.float32))).astype(np.float64)
    t = d["target"]
    saved = []
    for W in Ws:
        K = W.shape[1]
        g = O.absmean_gamma(W)
        q = O.ternary_codes(W, g)
        xq, s = O.act_quant(x)
        y = O.forward_y(O.forward_acc(xq, q), s, g)
        saved.append((xq, s, q, g, K))
        x = O.bf16_round(y)  # the layer output is written as bf16
    dY = O.bf16_round(x - t)
    grads = [None] * 3
    for i in (2, 1, 0):
        xq, s, q, g, K = saved[i]
        dX, dW = O.backward(dY, xq, s, q, g)
        grads[i] = dW
        dY = O.bf16_round(dX)  # identity STE through the activation quantizer
    # autograd on the quantised weights, same forward values
    Q = [torch.tensor(O.w_hat(q, g), requires_grad=True) for (_, _, q, g, _) in saved]
    a = torch.tensor(O.x_hat(saved[0][0], saved[0][1], saved[0][4]))
    for i in range(3):
        h = a @ Q[i].T
        if i < 2:
            xq, s, _, _, K = saved[i + 1]
            a = h + (torch.tensor(O.x_hat(xq, s, K)) - h).detach()
        else:
            a = h
    loss = 0.5 * torch.sum((a - torch.tensor(t)) ** 2)
    loss.backward()
    for i in range(3):
        assert np.array_equal(np.sign(grads[i]), np.sign(Q[i].grad.numpy())), i


# ---------------------------------------------------------------------------
# 1-bit sign gradients
# ---------------------------------------------------------------------------

def test_sign1_hand_bytes():
    """Row 0: negatives at k = 0, 4, 7, 8 (and -0.0 at k = 1, zero at k = 2,
    which are not negative): byte 0 = 1 + 16 + 128 = 0x91, byte 1 = 0x01.
    Row 1: the only negative at k = 2: byte 0 = 0x04. K = 10 pads to 64
    columns, 8 bytes per row; the padding bytes are 0."""
    d = np.array([[-1.0, -0.0, 0.0, 3.0, -2.0, 5.0, 6.0, -7.0, -1e-30, 2.0],
                  [1.0, 1.0, -4.0, 0.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0]])
    got = O.sign1_pack(d)
    want = np.zeros((2, 8), dtype=np.uint8)
    want[0, 0], want[0, 1], want[1, 0] = 0x91, 0x01, 0x04
    assert got.dtype == np.uint8 and np.array_equal(got, want)
    assert np.array_equal(O.sign1_unpack(got, 10), np.where(d < 0, -1, 1))


def test_sign1_matches_numpy_packbits():
    """Against numpy's own bit packing (little bit order) of dW < 0 on a
    random matrix with exact zeros, negative zeros and a ragged K."""
    rng = np.random.default_rng(5)
    for N, K in ((3, 1), (7, 70), (16, 128), (5, 1001)):
        d = rng.standard_normal((N, K))
        d[rng.random((N, K)) < 0.1] = 0.0
        d[rng.random((N, K)) < 0.1] = -0.0
        Kp = O.k_pad(K)
        full = np.zeros((N, Kp), dtype=bool)
        full[:, :K] = d < 0
        ref = np.packbits(full, axis=1, bitorder="little")
        got = O.sign1_pack(d)
        assert got.shape == (N, Kp // 8) and np.array_equal(got, ref), (N, K)
        assert int(np.unpackbits(got).sum()) == int(np.sum(d < 0))


def test_sign1_of_ste_gradient_matches_quantised_gradient():
    """The page's claim in its 1-bit form: on its 3-layer net through the
    oracle, the packed signs of the STE gradient equal the packed signs of
    autograd's gradient with respect to the quantised weights."""
    torch = pytest.importorskip("torch")
    d = WL.tiny_net_inputs()
    x = WL.bf16_bits_to_f32(WL.f32_to_bf16_bits(d["x0"].astype(np.float32))).astype(np.float64)
    saved = []
    for W in (w.astype(np.float32) for w in d["Ws"]):
        g = O.absmean_gamma(W)
        q = O.ternary_codes(W, g)
        xq, s = O.act_quant(x)
        saved.append((xq, s, q, g, W.shape[1]))
        x = O.bf16_round(O.forward_y(O.forward_acc(xq, q), s, g))
    dY = O.bf16_round(x - d["target"])
    grads = [None] * 3
    for i in (2, 1, 0):
        xq, s, q, g, K = saved[i]
        dX, grads[i] = O.backward(dY, xq, s, q, g)
        dY = O.bf16_round(dX)
    Q = [torch.tensor(O.w_hat(q, g), requires_grad=True) for (_, _, q, g, _) in saved]
    a = torch.tensor(O.x_hat(saved[0][0], saved[0][1], saved[0][4]))
    for i in range(3):
        h = a @ Q[i].T
        if i < 2:
            xq, s, _, _, K = saved[i + 1]
            a = h + (torch.tensor(O.x_hat(xq, s, K)) - h).detach()
        else:
            a = h
    (0.5 * torch.sum((a - torch.tensor(d["target"])) ** 2)).backward()
    for i in range(3):
        gq = Q[i].grad.numpy()
        assert np.all(gq != 0), i  # every sign is determined
        assert np.array_equal(O.sign1_pack(grads[i]), O.sign1_pack(gq)), i


# ---------------------------------------------------------------------------
# the synthetic weight recipe
# ---------------------------------------------------------------------------

def test_kaiming_bound_matches_printed_init():
    """The 200 printed master weights of a fresh 10 -> 20 layer lie inside
    +-1/sqrt(fan_in) and reach 0.99 of it: U(+-1/sqrt(fan_in)) is the init
    bound used for the synthetic weights."""
    vals = np.loadtxt(os.path.join(GOLDEN, "bitlinearnew_init_weights_20x10.txt"))
    assert vals.shape == (20, 10)
    b = 1.0 / math.sqrt(10)
    assert np.all(np.abs(vals) <= b)
    assert np.max(np.abs(vals)) > 0.99 * b
    d = WL.custom_inputs(8, 10, 20)
    w = WL.bf16_bits_to_f32(d["W"])
    assert np.all(np.abs(w) <= b * (1 + 2 ** -8))


# ---------------------------------------------------------------------------
# TTQ ("TTQ_VERIFICATION.md")
# ---------------------------------------------------------------------------

def rne_f32(fr):
    """Round a nonzero Fraction in the normal fp32 range to 24 significant
    bits, ties to even."""
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 2 ** 24:
        a /= 2
        e += 1
    while a < 2 ** 23:
        a *= 2
        e -= 1
    return sgn * Fraction(rne_int(a)) * (Fraction(2) ** e)


def test_ttq_init_hand_example():
    """Initialization (Eq. 2): W = [0.75, -0.25, 0.125, -0.5] has E|W| =
    1.625 / 4 = 0.40625 (exact), so Wp = Wn = 0.40625 and delta is
    0.7 (as fp32) times 0.40625, rounded once to fp32; with that delta the
    codes of Eq. 1 are [+1, 0, 0, -1]."""
    w = np.array([[0.75, -0.25, 0.125, -0.5]], dtype=np.float32)
    delta, wp, wn = O.ttq_init(w)
    assert float(wp) == 0.40625 and float(wn) == 0.40625
    expect = rne_f32(Fraction(float(np.float32(0.7))) * Fraction(13, 32))
    assert Fraction(float(delta)) == expect
    assert 0.28 < float(delta) < 0.29
    assert O.ttq_codes(w, delta).tolist() == [[1, 0, 0, -1]]


def test_ttq_init_is_point_seven_of_mean_abs():
    """delta / E stays within one fp32 rounding of 0.7, and E is the
    exactly rounded mean of |W| (compared with a Fraction sum), over
    random bf16 and fp32 weights of several sizes."""
    rng = np.random.default_rng(31)
    for shape in ((3, 5), (17, 64), (64, 130)):
        w = rng.standard_normal(shape).astype(np.float32) * 0.02
        delta, wp, wn = O.ttq_init(w)
        exact = sum(Fraction(float(v)) for v in np.abs(w).ravel()) / w.size
        assert Fraction(float(wp)) == rne_f32(exact) and wp == wn
        assert Fraction(float(delta)) == rne_f32(Fraction(float(np.float32(0.7))) * Fraction(float(wp)))


def test_ttq_codes_strict_threshold():
    """Eq. 1 is strict on both sides: |w| == delta gives 0, the next fp32
    value above gives +-1; brute force against exact comparisons of
    Fractions on random values near the threshold."""
    d = np.float32(0.3)
    up = np.nextafter(d, np.float32(1))
    dn = np.nextafter(d, np.float32(0))
    w = np.array([[d, -d, up, -up, dn, -dn, 0.0, 5.0, -5.0]], dtype=np.float32)
    assert O.ttq_codes(w, d).tolist() == [[0, 0, 1, -1, 0, 0, 0, 1, -1]]
    rng = np.random.default_rng(37)
    w = (np.float32(0.3) + rng.integers(-3, 4, (40, 9)).astype(np.float32) * np.float32(2 ** -25)) \
        * rng.choice([-1, 1], (40, 9)).astype(np.float32)
    q = O.ttq_codes(w, d)
    fd = Fraction(float(d))
    for (i, j), v in np.ndenumerate(w):
        fv = Fraction(float(v))
        assert q[i, j] == (1 if fv > fd else -1 if fv < -fd else 0), (v, q[i, j])


def test_ttq_values_hand():
    """Values of Eq. 1 in bf16: code +1 -> bf16(Wp), -1 -> -bf16(Wn), 0 -> 0,
    with the bf16 rounding taken from exact Fraction arithmetic."""
    wp, wn = np.float32(0.3), np.float32(0.7)
    v = O.ttq_values(np.array([[1, 0, -1, 1]]), wp, wn)
    p = float(rne_bf16(Fraction(float(wp))))
    n = float(rne_bf16(Fraction(float(wn))))
    assert v.tolist() == [[p, 0.0, -n, p]]
    assert p != float(wp) and n != float(wn)  # the rounding is not a no-op here


def test_ttq_against_torch_autograd():
    """Independent route: Eq. 1 written with torch.where on leaf tensors Wp
    and Wn and an identity straight-through path to W (W_q + W - W.detach()),
    in torch float64 on the CPU. Autograd's gradients of x, W, Wp and Wn
    equal the oracle's dX, dW, grad_Wp and grad_Wn, and y matches."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    M, K, N = 12, 40, 18
    x = bf16_vals(rng, (M, K))
    w = bf16_vals(rng, (N, K), 0.05)
    dY = bf16_vals(rng, (M, N))
    wp, wn, delta = np.float32(0.046875), np.float32(0.03515625), np.float32(0.035)  # Wp, Wn bf16-exact
    r = O.ttq_layer(x, w, dY, params=(delta, wp, wn))
    xt = torch.tensor(x, requires_grad=True)
    W = torch.tensor(w, requires_grad=True)
    tp = torch.tensor(float(wp), dtype=torch.float64, requires_grad=True)
    tn = torch.tensor(float(wn), dtype=torch.float64, requires_grad=True)
    d = float(delta)
    zero = torch.zeros((), dtype=torch.float64)
    wq = torch.where(W > d, tp, torch.where(W < -d, -tn, zero))
    y = torch.nn.functional.linear(xt, wq + W - W.detach())
    y.backward(torch.tensor(dY))
    assert np.allclose(y.detach().numpy(), r["y"], rtol=1e-12, atol=1e-14)
    assert np.allclose(xt.grad.numpy(), r["dX"], rtol=1e-12, atol=1e-14)
    assert np.allclose(W.grad.numpy(), r["dW"], rtol=1e-12, atol=1e-14)
    assert math.isclose(tp.grad.item(), r["g_wp"], rel_tol=1e-12, abs_tol=1e-12)
    assert math.isclose(tn.grad.item(), r["g_wn"], rel_tol=1e-12, abs_tol=1e-12)
    assert (r["q"] == 1).any() and (r["q"] == -1).any() and (r["q"] == 0).any()


def test_ttq_reduces_to_bitnet_quantizer():
    """With Wp = Wn = gamma and delta = gamma / 2 (exact in fp32), TTQ's codes
    are the BitNet RoundClip codes (ties at |w| = gamma/2 go to 0 in both),
    its values are q * bf16(gamma) and its dX is the BitNet STE dX."""
    w = np.array([[1.0, -0.5, 0.25, -0.25]], dtype=np.float32)
    g = O.absmean_gamma(w)
    assert float(g) == 0.5  # so +-0.25 sit exactly at gamma / 2
    half = np.float32(g / np.float32(2))
    q = O.ttq_codes(w, half)
    assert q.tolist() == [[1, -1, 0, 0]]
    assert np.array_equal(q, O.ternary_codes(w, g))
    assert np.array_equal(O.ttq_values(q, g, g), O.w_hat(q, g))
    rng = np.random.default_rng(43)
    w = bf16_vals(rng, (24, 70), 0.05)
    g = O.absmean_gamma(w)
    half = np.float32(g / np.float32(2))
    q = O.ttq_codes(w, half)
    assert np.array_equal(q, O.ternary_codes(w, g))
    dY = bf16_vals(rng, (9, 24))
    x = bf16_vals(rng, (9, 70))
    dX_ttq = O.ttq_backward(dY, x, q, g, g)[0]
    x_q, s = O.act_quant(x)
    dX_bitnet = O.backward(dY, x_q, s, q, g)[0]
    assert np.array_equal(dX_ttq, dX_bitnet)


def test_ttq_grads_exact_fractions():
    """With small-integer dY and x every dW entry is an exact integer: the
    oracle's dW, grad_Wp and grad_Wn equal Python integer sums (ragged
    shapes; the codes pattern from random signs)."""
    rng = np.random.default_rng(47)
    for M, N, K in ((5, 3, 7), (33, 17, 65), (64, 40, 130)):
        dY = rng.integers(-3, 4, (M, N)).astype(np.float64)
        x = rng.integers(-3, 4, (M, K)).astype(np.float64)
        q = rng.integers(-1, 2, (N, K)).astype(np.int8)
        dX, dW, g_wp, g_wn = O.ttq_backward(dY, x, q, np.float32(0.5), np.float32(0.25))
        dYi = dY.astype(np.int64)
        xi = x.astype(np.int64)
        dWi = [[sum(int(dYi[m, n]) * int(xi[m, k]) for m in range(M)) for k in range(K)] for n in range(N)]
        assert dW.tolist() == [[float(v) for v in row] for row in dWi]
        ep = sum(dWi[n][k] for n in range(N) for k in range(K) if q[n, k] == 1)
        en = -sum(dWi[n][k] for n in range(N) for k in range(K) if q[n, k] == -1)
        assert g_wp == float(ep) and g_wn == float(en)
        # dX on exact values: 0.5 and 0.25 are bf16-exact
        ex = [[sum(int(dYi[m, n]) * Fraction(0.5 if q[n, k] == 1 else -0.25 if q[n, k] == -1 else 0)
                   for n in range(N)) for k in range(K)] for m in range(M)]
        assert dX.tolist() == [[float(v) for v in row] for row in ex]
