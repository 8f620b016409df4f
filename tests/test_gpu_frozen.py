"""The frozen (inference) path of the BitNet layer on the GPU, through the C
ABI: ``QATBitLinear.freeze`` / ``unfreeze``, ``export_inference``, the
forward from a stored (w_packed, gamma) (``bitlinear_inference``) and
``ternary_stats`` ("bitlinear.py", BitLinear.freeze, unfreeze,
_inference_mode and ternary_stats; "bitnet-qat-train", Usage:
export_inference returns the packed weights and their scale).

Checked against the oracle: the exported bytes and gamma bit for bit, the
frozen forward's y within the bar (its accumulator is exact), the code
counts exactly; and against the training path: a frozen forward equals the
training forward at the moment of freezing bit for bit, and so does its dX.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import compare as C
from ternary_weight_quantization_amd import workloads as WL
from tests.gpu_util import dev_bf16, host_bf16_bits, note, w_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from ternary_weight_quantization_amd import binding
    binding.lib()


def bf(bits):
    return WL.bf16_bits_to_f32(bits).astype(np.float64)


def _layer(inp):
    from ternary_weight_quantization_amd.layer import QATBitLinear
    K, N = inp["K"], inp["N"]
    layer = QATBitLinear(K, N, device="cuda", dtype=torch.bfloat16)
    with torch.no_grad():
        layer.weight.copy_(dev_bf16(inp["W"]))
    return layer


@pytest.mark.parametrize("M", [1, 32, 64, 4096])
def test_frozen_forward_matches_training_and_oracle(M):
    """K = 2560, N = 6912 (the up-projection) at M = 1, 32, 64 (the
    few-token kernels) and 4096 (the large-M GEMM; oracle on sampled
    elements)."""
    K, N = 2560, 6912
    inp = WL.custom_inputs(M, K, N, seed=100 + M)
    note(f"frozen forward M={M} K={K} N={N}")
    layer = _layer(inp)
    x = dev_bf16(inp["x"])
    y_train = host_bf16_bits(layer(x).detach())
    layer.freeze()
    assert layer.frozen and "frozen=True" in repr(layer)
    wp, gamma = layer.export_inference()
    # the cached state is returned, not recomputed
    assert wp.data_ptr() == layer.export_inference()[0].data_ptr()
    w = w_values(inp["W"])
    g_ref = O.absmean_gamma(w)
    q = O.ternary_codes(w, g_ref)
    assert np.float32(gamma.item()).view(np.uint32) == np.float32(g_ref).view(np.uint32)
    assert np.array_equal(wp.cpu().numpy(), O.pack_codes(q, O.k_pad(K)))
    # master updates do not reach a frozen layer
    with torch.no_grad():
        layer.weight.mul_(-1.0)
    y_frozen = host_bf16_bits(layer(x).detach())
    assert np.array_equal(y_frozen, y_train)
    from ternary_weight_quantization_amd.layer import bitlinear_inference
    y_exp = host_bf16_bits(bitlinear_inference(x, wp, gamma, K).detach())
    assert np.array_equal(y_exp, y_train)
    x_q, s = O.act_quant(bf(inp["x"]), O.k_pad(K))
    if M <= 64:
        m = C.check(bf(y_frozen), O.forward_y(O.forward_acc(x_q, q), s, g_ref), "y")
    else:
        rng = np.random.default_rng(M)
        r, c = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
        m = C.check(bf(y_frozen)[r, c], O.y_elements(x_q, s, q, g_ref, r, c), "y")
    note(f"  frozen y max_rel {m['max_rel']:.2e} normwise {m['normwise']:.2e}")
    # unfreezing goes back to the masters (now negated: y changes sign)
    layer.unfreeze()
    assert not layer.frozen
    y_neg = host_bf16_bits(layer(x).detach())
    assert np.array_equal(bf(y_neg), -bf(y_train))


@pytest.mark.parametrize("M,K,N", [(32, 2560, 6912), (300, 1000, 776)])
def test_frozen_backward_gives_dx_only(M, K, N):
    """A frozen layer is differentiable in x: dX equals the training layer's
    dX bit for bit (the same kernels on the same 2-bit state) and matches the
    oracle; the masters get no gradient."""
    inp = WL.custom_inputs(M, K, N, seed=7 + M)
    note(f"frozen backward M={M} K={K} N={N}")
    layer = _layer(inp)
    dY = dev_bf16(inp["dY"])
    x1 = dev_bf16(inp["x"]).requires_grad_(True)
    layer(x1).backward(dY)
    layer.weight.grad = None
    layer.freeze()
    x2 = dev_bf16(inp["x"]).requires_grad_(True)
    layer(x2).backward(dY)
    assert layer.weight.grad is None
    assert np.array_equal(host_bf16_bits(x2.grad), host_bf16_bits(x1.grad))
    w = w_values(inp["W"])
    g = O.absmean_gamma(w)
    q = O.ternary_codes(w, g)
    x_q, s = O.act_quant(bf(inp["x"]), O.k_pad(K))
    dX_ref, _ = O.backward(bf(inp["dY"]), x_q, s, q, g)
    C.check(bf(host_bf16_bits(x2.grad)), dX_ref, "dX")


@pytest.mark.parametrize("name", ["c1_small", "c2_up_4096x2560x6912", "c5_skinny_32x6912x2560"])
def test_ternary_stats_counts_exact(name):
    """The shares of -1, 0, +1 reported next to parity: the GPU counts equal
    the oracle's codes exactly. C2 has U(+-a) weights (zero share about 1/4),
    C5 N(0, 0.02) with 10 % exact zeros (about 0.352)."""
    from ternary_weight_quantization_amd.layer import QATBitLinear
    inp = WL.layer_inputs(name, seed=0)
    K, N = inp["K"], inp["N"]
    note(f"ternary stats {name}")
    dt = torch.float32 if inp["w_dtype"] == "f32" else torch.bfloat16
    layer = QATBitLinear(K, N, device="cuda", dtype=dt)
    with torch.no_grad():
        layer.weight.copy_(dev_bf16(inp["W"]) if dt == torch.bfloat16 else torch.from_numpy(inp["W"]).cuda())
    st = layer.ternary_stats
    w = w_values(inp["W"])
    q = O.ternary_codes(w, O.absmean_gamma(w))
    n = N * K
    assert round(st["neg1"] * n) == int(np.sum(q == -1))
    assert round(st["pos1"] * n) == int(np.sum(q == 1))
    assert round(st["zero"] * n) == int(np.sum(q == 0))
    note(f"  {name}: -1 {st['neg1']:.4f}  0 {st['zero']:.4f}  +1 {st['pos1']:.4f}")
    if name == "c2_up_4096x2560x6912":
        assert abs(st["zero"] - 0.25) < 0.005
    if name == "c5_skinny_32x6912x2560":
        assert abs(st["zero"] - 0.352) < 0.005
    layer.freeze()
    assert layer.ternary_stats == st
