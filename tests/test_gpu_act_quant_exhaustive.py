"""Exhaustive check of the GPU activation quantizer's rounding ("bitlinear.py",
activation_quant_int8; "1BitTraining.md", activation_quant: x_q =
clip(round_half_even(127 x / s), -127, 127) with s the row absmax).

Every bf16 significand of the scale s in [1, 2) against every bf16
significand of x in the nine binades from [1/256, 1/128) to [1, 2) with
x <= s (smaller x give 127 x / s < 1/2, so 0 with no rounding question):
139,328 pairs [s, x]. The answer depends only on the two
significands and the exponent gap, so this covers every rounding decision a
bf16 row can ask for. The kernel takes rint(x * fl(127/s)) unless the
product lies within 2^-15 of a half-integer, and recomputes those in fp64;
this set holds the pairs where the reciprocal product alone rounds wrongly
and every exact tie (rows whose s has significand 254/128). Checked bit for
bit against exact integer arithmetic and against the oracle, through
bitnet_act_quant, in each kernel layout the library picks by row length.
"""

import numpy as np
import pytest
import torch

import oracle as O
from ternary_weight_quantization_amd import workloads as WL
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


def _pairs():
    sig = np.arange(128, 256, dtype=np.int64)          # 8-bit significands
    S = np.repeat(sig, 128 * 9)                       # s = S / 128
    X = np.tile(np.tile(sig, 9), 128)                 # x = X / 128 * 2^-d
    D = np.tile(np.repeat(np.arange(9), 128), 128)
    keep = (X * 2.0 ** -D) <= S
    S, X, D = S[keep], X[keep], D[keep]
    num, den = 127 * X, S << D
    q = num // den
    r = num - q * den
    want = q + ((2 * r > den) | ((2 * r == den) & (q % 2 == 1)))
    return S / 128.0, X / 128.0 * 2.0 ** -D, want


def _run(rows_f32, K):
    from ternary_weight_quantization_amd import binding as B
    M = rows_f32.shape[0]
    bits = WL.f32_to_bf16_bits(rows_f32)
    assert np.array_equal(WL.bf16_bits_to_f32(bits), rows_f32)  # the values are bf16-exact
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    x_q = torch.empty((M, B.bitnet_k_pad(K)), dtype=torch.int8, device="cuda")
    s = torch.empty((M,), dtype=torch.float32, device="cuda")
    B.bitnet_act_quant(x, x_q, s)
    torch.cuda.synchronize()
    return x_q.cpu().numpy(), s.cpu().numpy()


def test_pair_set_holds_reciprocal_failures_and_ties():
    """The set exercises the recompute path: the fp32 reciprocal product
    alone (numpy float32) rounds some pairs wrongly, and exact ties exist."""
    s, x, want = _pairs()
    assert len(want) == 139_328
    r127 = (np.float32(127.0) / s.astype(np.float32)).astype(np.float32)
    p = (x.astype(np.float32) * r127).astype(np.float32)
    assert int(np.sum(np.rint(p).astype(np.int64) != want)) >= 1
    t = 127.0 * x / s
    assert int(np.sum(t - np.floor(t) == 0.5)) >= 1


@pytest.mark.parametrize("scale_exp", [-100, -26, -20, 0, 20, 100])
def test_act_quant_exhaustive_pairs_gpu(scale_exp):
    """Rows [s, x] (K = 2): s is the row's absmax, so x_q[:, 0] = 127 and
    x_q[:, 1] = RNE(127 x / s). A common power of two 2^e leaves every
    decision unchanged (fl(127/s) scales exactly), so each e with s >= 1e-8
    must give the same codes. At e = -100 every row's absmax is below the
    1e-8 floor, so s = 1e-8 and the codes are those of the oracle, whose
    floor is the same."""
    s, x, want = _pairs()
    f = 2.0 ** scale_exp
    rows = np.stack([s * f, x * f], axis=1).astype(np.float32)
    note(f"act-quant exhaustive pairs, scale 2^{scale_exp}, {rows.shape[0]} rows")
    xq, sg = _run(rows, 2)
    oq, os_ = O.act_quant(rows.astype(np.float64), xq.shape[1])
    assert np.array_equal(oq, xq) and np.array_equal(os_.view(np.uint32), sg.view(np.uint32))
    assert np.all(xq[:, 2:] == 0)
    if (s * f).min() >= 1e-8:
        assert np.array_equal(sg.view(np.uint32), (s * f).astype(np.float32).view(np.uint32))
        assert np.all(xq[:, 0] == 127)
        assert np.array_equal(xq[:, 1].astype(np.int64), want)
    else:
        assert np.all(sg == np.float32(1e-8))


@pytest.mark.parametrize("K", [1153, 8200, 18000])
def test_act_quant_exhaustive_long_rows_gpu(K):
    """The same pairs grouped by scale: one row per significand of s, s at
    column 0 and its up to 1,152 x (signs alternating) after it, zeros
    after that. K = 1153 (not a multiple of 8: element loads), 8200 (the
    register-resident layout with more threads per row) and 18000 (the
    two-pass long-row kernel)."""
    s, x, want = _pairs()
    sig = np.round(s * 128).astype(np.int64)
    rows = np.zeros((128, K), dtype=np.float32)
    exp = np.zeros((128, K), dtype=np.int64)
    for i, v in enumerate(range(128, 256)):
        sel = np.nonzero(sig == v)[0]
        xs = x[sel] * np.where(np.arange(len(sel)) % 2 == 0, 1.0, -1.0)
        rows[i, 0] = v / 128.0
        rows[i, 1:1 + len(sel)] = xs
        exp[i, 0] = 127
        exp[i, 1:1 + len(sel)] = want[sel] * np.where(np.arange(len(sel)) % 2 == 0, 1, -1)
    note(f"act-quant exhaustive long rows K={K}")
    xq, sg = _run(rows, K)
    assert np.array_equal(sg, (np.arange(128, 256) / 128.0).astype(np.float32))
    assert np.array_equal(xq[:, :K].astype(np.int64), exp)
    assert np.all(xq[:, K:] == 0)


@pytest.mark.parametrize("K", [1216, 7168])
def test_act_quant_exhaustive_through_quantize_gpu(K):
    """The long rows above through bitnet_quantize with a bf16 weight and K a
    multiple of 64, so that the one-pass launch quantizes them (64 threads x
    3 chunks per row at K = 1216, 128 x 7 at K = 7168) next to the weight:
    every code and scale bit for bit, and the weight's outputs as the
    oracle's."""
    from ternary_weight_quantization_amd import binding as B
    s, x, want = _pairs()
    sig = np.round(s * 128).astype(np.int64)
    rows = np.zeros((128, K), dtype=np.float32)
    exp = np.zeros((128, K), dtype=np.int64)
    for i, v in enumerate(range(128, 256)):
        sel = np.nonzero(sig == v)[0]
        xs = x[sel] * np.where(np.arange(len(sel)) % 2 == 0, 1.0, -1.0)
        rows[i, 0] = v / 128.0
        rows[i, 1:1 + len(sel)] = xs
        exp[i, 0] = 127
        exp[i, 1:1 + len(sel)] = want[sel] * np.where(np.arange(len(sel)) % 2 == 0, 1, -1)
    N = 40
    W_bits = WL.custom_inputs(1, K, N, seed=K, w_dtype="bf16")["W"]
    note(f"act-quant exhaustive rows through bitnet_quantize K={K}")
    bits = WL.f32_to_bf16_bits(rows)
    xd = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    Wd = torch.from_numpy(np.ascontiguousarray(W_bits).view(np.int16)).cuda().view(torch.bfloat16)
    Kp = B.bitnet_k_pad(K)
    w_packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device="cuda")
    gamma = torch.empty((1,), dtype=torch.float32, device="cuda")
    x_q = torch.empty((128, Kp), dtype=torch.int8, device="cuda")
    s_x = torch.empty((128,), dtype=torch.float32, device="cuda")
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device="cuda")
    B.bitnet_quantize(Wd, xd, w_packed, gamma, x_q, s_x, ws)
    torch.cuda.synchronize()
    xq, sg = x_q.cpu().numpy(), s_x.cpu().numpy()
    assert np.array_equal(sg, (np.arange(128, 256) / 128.0).astype(np.float32))
    assert np.array_equal(xq[:, :K].astype(np.int64), exp)
    w = WL.bf16_bits_to_f32(W_bits).astype(np.float64)
    g = O.absmean_gamma(w)
    assert np.float32(gamma.item()).view(np.uint32) == np.float32(g).view(np.uint32)
    assert np.array_equal(w_packed.cpu().numpy(), O.pack_codes(O.ternary_codes(w, g), Kp))
