"""GPU parity of the TTQ path ("TTQ_VERIFICATION.md") against the CPU oracle,
through the C ABI.

Bit-exact: the initial (delta, Wp, Wn), the 2-bit codes and the bf16 weight
values. Within tolerance (``oracle.compare`` with the 2^-8 RMS floor: the
products are fp32 sums of bf16 products, which can cancel): y, dX, dW. The
scale gradients are fp32 sums (per 128 x 128 tile, then fp64 across tiles)
of the fp32 dW values; their error is bounded by the recursive-summation
bound (M + 512) * 2^-24 * B, B = the sum over the masked positions of
sum_m |dY[m, n] x[m, k]|, and they are exact for integer-valued inputs.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import compare as C
from ternary_weight_quantization_amd import workloads as WL
from tests.gpu_util import note, run_ttq, w_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from ternary_weight_quantization_amd import binding
    binding.lib()


def bf(bits):
    return WL.bf16_bits_to_f32(bits).astype(np.float64)


def f32_bits(v):
    return np.float32(v).view(np.uint32)


def grads_bound(dY, x, q, M):
    """(M + 512) * 2^-24 * B for the +1 and the -1 masks."""
    B = np.abs(dY).T @ np.abs(x)
    u = 2.0 ** -24 * (M + 512)
    return u * float(B[q == 1].sum()), u * float(B[q == -1].sum())


def check_ttq(inp, g, given=None):
    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = O.k_pad(K)
    w = w_values(inp["W"])
    x = bf(inp["x"])
    dY = bf(inp["dY"])
    if given is None:
        delta, wp, wn = O.ttq_init(w)
        assert [f32_bits(v) for v in g["params"]] == [f32_bits(delta), f32_bits(wp), f32_bits(wn)], \
            (g["params"], (delta, wp, wn))
    else:
        delta, wp, wn = (np.float32(v) for v in given)
    q = O.ttq_codes(w, delta)
    assert np.array_equal(g["packed"], O.pack_codes(q, Kp))
    wt = O.ttq_values(q, wp, wn)
    wt_bits = np.zeros((N, Kp), dtype=np.uint16)
    wt_bits[:, :K] = WL.f32_to_bf16_bits(wt.astype(np.float32))
    assert np.array_equal(g["wt_bits"], wt_bits)
    out = {"y": C.check(bf(g["y_bits"]), O.ttq_forward(x, wt), "y_ttq")}
    dX, dW, g_wp, g_wn = O.ttq_backward(dY, x, q, wp, wn)
    if "dX" in g:
        out["dX"] = C.check(g["dX"], dX, "dX")
    if "dW" in g:
        out["dW"] = C.check(g["dW"], dW, "dW")
    if "grads" in g:
        bp, bn = grads_bound(dY, x, q, M)
        # the bound plus the final rounding to fp32
        assert abs(float(g["grads"][0]) - g_wp) <= bp + 2.0 ** -24 * abs(g_wp), (g["grads"], g_wp, bp)
        assert abs(float(g["grads"][1]) - g_wn) <= bn + 2.0 ** -24 * abs(g_wn), (g["grads"], g_wn, bn)
        out["grads"] = (float(g["grads"][0]), g_wp, float(g["grads"][1]), g_wn)
    print(f"[ttq parity] M={M} K={K} N={N}: " + ", ".join(
        f"{k}=max_rel {v['max_rel']:.2e} norm {v['normwise']:.2e}" if isinstance(v, dict) else f"{k}={v}"
        for k, v in out.items()), flush=True)
    fr = np.array([np.mean(q == 1), np.mean(q == 0), np.mean(q == -1)])
    print(f"[ttq stats] fractions +1/0/-1: {fr.round(3).tolist()}", flush=True)
    return out


@pytest.mark.parametrize("M,K,N,wd", [
    (1, 1, 1, "bf16"),
    (2, 7, 6, "f32"),
    (64, 256, 128, "f32"),
    (257, 320, 200, "bf16"),
    (300, 1001, 777, "bf16"),
    (33, 130, 513, "f32"),
    (520, 1000, 264, "bf16"),
    (1024, 512, 96, "bf16"),
])
def test_ttq_ragged_shapes(M, K, N, wd):
    inp = WL.custom_inputs(M, K, N, seed=3 * M + K + N, w_dtype=wd)
    note(f"ttq ragged M={M} K={K} N={N} W={wd}")
    check_ttq(inp, run_ttq(inp))


@pytest.mark.parametrize("dw_f32", [False, True])
def test_ttq_given_params(dw_f32):
    """Asymmetric Wp != Wn and a threshold that is not 0.7 E (the values a
    trained layer holds), neither bf16-exact; dW in bf16 and in f32."""
    inp = WL.custom_inputs(384, 576, 320, seed=11)
    w = w_values(inp["W"])
    e = float(np.mean(np.abs(w)))
    params = (np.float32(0.55 * e), np.float32(1.37 * e), np.float32(0.81 * e))
    note(f"ttq given params {params} dW f32={dw_f32}")
    check_ttq(inp, run_ttq(inp, params=params, dw_f32=dw_f32), given=params)


def test_ttq_grads_exact_for_integer_inputs():
    """Integer-valued x and dY (|v| <= 3) make every dW entry, every partial
    and every total an exact integer in fp32: grads, and the f32 dW, equal the
    oracle exactly. Codes from random weights in {-1, -0.25, 0, 0.25, 1}."""
    M, K, N = 320, 520, 300
    rng = np.random.default_rng(23)
    inp = WL.custom_inputs(M, K, N, seed=23)
    inp["x"] = WL.f32_to_bf16_bits(rng.integers(-3, 4, (M, K)).astype(np.float32))
    inp["dY"] = WL.f32_to_bf16_bits(rng.integers(-3, 4, (M, N)).astype(np.float32))
    inp["W"] = WL.f32_to_bf16_bits(rng.choice([-1.0, -0.25, 0.0, 0.25, 1.0], (N, K)).astype(np.float32))
    params = (np.float32(0.5), np.float32(0.75), np.float32(0.375))
    note("ttq integer inputs")
    g = run_ttq(inp, params=params, dw_f32=True)
    x, dY = bf(inp["x"]), bf(inp["dY"])
    q = O.ttq_codes(w_values(inp["W"]), params[0])
    dX, dW, g_wp, g_wn = O.ttq_backward(dY, x, q, params[1], params[2])
    assert np.array_equal(g["dW"], dW)
    assert float(g["grads"][0]) == g_wp and float(g["grads"][1]) == g_wn, (g["grads"], g_wp, g_wn)
    # y: exact fp32 sums (multiples of 1/8 below 2^11), rounded once to bf16
    assert np.array_equal(bf(g["y_bits"]), O.bf16_round(O.ttq_forward(x, O.ttq_values(q, *params[1:]))))


def test_ttq_edge_all_zero_weight():
    """All-zero W: E is floored at 1e-8 as gamma is, delta = fl32(0.7 * 1e-8);
    every code is 0 (|0| > delta fails), so wt, y and dX are zero and the
    scale gradients are 0."""
    inp = WL.custom_inputs(64, 192, 96, seed=5)
    inp["W"] = np.zeros_like(inp["W"])
    note("ttq edge: all-zero W")
    g = run_ttq(inp)
    assert f32_bits(g["params"][1]) == f32_bits(np.float32(1e-8))
    assert np.all(g["packed"] == 0) and np.all(g["wt_bits"] == 0)
    assert np.all(g["y_bits"] == 0) and np.all(g["dX"] == 0)
    assert np.all(g["grads"] == 0)
    check_ttq(inp, g)


def test_ttq_optional_outputs():
    """dX alone, dW alone (with and without the scale gradients) give the
    same values as the full call."""
    inp = WL.custom_inputs(200, 320, 136, seed=29)
    note("ttq optional outputs")
    full = run_ttq(inp)
    a = run_ttq(inp, dw=False, grads=False)
    b = run_ttq(inp, dx=False)
    c = run_ttq(inp, dx=False, grads=False)
    assert np.array_equal(a["dX"], full["dX"])
    assert np.array_equal(b["dW"], full["dW"]) and np.array_equal(c["dW"], full["dW"])
    assert np.array_equal(b["grads"].view(np.uint32), full["grads"].view(np.uint32))


@pytest.mark.parametrize("knob", [None, "-1"])
def test_ttq_paired_backward(set_knobs, knob):
    """2048 x 1024 -> 1024: dX and dW split their tiles, so they run in one
    paired launch; the split_ctas knob at -1 forces whole tiles,
    one product after the other. Both against the oracle."""
    if knob is not None:
        set_knobs(split_ctas=int(knob))
    inp = WL.custom_inputs(2048, 1024, 1024, seed=31)
    note(f"ttq paired backward, split_ctas={knob}")
    check_ttq(inp, run_ttq(inp))


@pytest.mark.parametrize("name", ["c2_up_4096x2560x6912", "c3_down_4096x6912x2560"])
def test_ttq_full_size_sampled(name):
    """The 4096 x 2560 -> 6912 layer (in the launch configuration the
    benchmark times) and the 4096 x 6912 -> 2560 one: bit-exact parameters,
    codes and values; y, dX, dW on sampled elements; the scale gradients
    against the masked sums of the GPU's own f32 dW (a property at any
    size), and that f32 dW sampled against the oracle."""
    inp = WL.layer_inputs(name, seed=0)
    M, K, N = inp["M"], inp["K"], inp["N"]
    note(f"ttq full size M={M} K={K} N={N}")
    g = run_ttq(inp, dw_f32=True)
    w = w_values(inp["W"])
    delta, wp, wn = O.ttq_init(w)
    assert [f32_bits(v) for v in g["params"]] == [f32_bits(delta), f32_bits(wp), f32_bits(wn)]
    q = O.ttq_codes(w, delta)
    assert np.array_equal(g["packed"], O.pack_codes(q))
    wt = O.ttq_values(q, wp, wn)
    assert np.array_equal(g["wt_bits"][:, :K], WL.f32_to_bf16_bits(wt.astype(np.float32)))
    x, dY = bf(inp["x"]), bf(inp["dY"])
    rng = np.random.default_rng(7)
    n = 4000
    r, c = rng.integers(0, M, n), rng.integers(0, N, n)
    C.check(bf(g["y_bits"])[r, c], O.ttq_y_elements(x, wt, r, c), "y_ttq")
    rk = rng.integers(0, K, n)
    C.check(g["dX"][r, rk], O.ttq_dx_elements(dY, wt, r, rk), "dX")
    rn, rk2 = rng.integers(0, N, n), rng.integers(0, K, n)
    C.check(g["dW"][rn, rk2], O.ttq_dw_elements(dY, x, rn, rk2), "dW")
    dW = g["dW"]
    sp = math.fsum(dW[q == 1].tolist())
    sn = -math.fsum(dW[q == -1].tolist())
    # the kernel sums the same fp32 values (the f32 store is exact): 256 per
    # lane in order, then a 6-level butterfly over the wave, then fp64, so
    # the error is within (256 + 6 + 1) * 2^-24 of the sum of |values|
    tol_p = 263 * 2.0 ** -24 * float(np.abs(dW[q == 1]).sum())
    tol_n = 263 * 2.0 ** -24 * float(np.abs(dW[q == -1]).sum())
    assert abs(float(g["grads"][0]) - sp) <= tol_p + 2.0 ** -24 * abs(sp), (g["grads"], sp, tol_p)
    assert abs(float(g["grads"][1]) - sn) <= tol_n + 2.0 ** -24 * abs(sn), (g["grads"], sn, tol_n)
    print(f"[ttq full] grads {g['grads'].tolist()} vs sums of dW {sp:.6g} {sn:.6g}", flush=True)


def test_ttq_module():
    """TTQLinear: the forward and the gradients of x, the weight and the raw
    scale parameters (softplus chain) against the oracle on the parameters
    the module passes."""
    from ternary_weight_quantization_amd.ttq_layer import TTQLinear
    torch.manual_seed(0)
    M, K, N = 96, 320, 200
    note("ttq module")
    layer = TTQLinear(K, N)
    p = layer.params().detach().cpu().numpy()
    w = layer.weight.detach().float().cpu().numpy().astype(np.float64)
    delta0, e0, _ = O.ttq_init(w)
    # after the softplus round trip the scales are within a few ulps of Eq. 2
    assert np.allclose(p, [delta0, e0, e0], rtol=1e-5)
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16).requires_grad_(True)
    y = layer(x)
    dy = torch.randn(M, N, device="cuda").to(torch.bfloat16)
    y.backward(dy)
    xs = x.detach().float().cpu().numpy().astype(np.float64)
    dys = dy.float().cpu().numpy().astype(np.float64)
    r = O.ttq_layer(xs, w, dys, params=tuple(np.float32(v) for v in p))
    C.check(y.detach().float().cpu().numpy(), r["y"], "y_ttq")
    C.check(x.grad.float().cpu().numpy(), r["dX"], "dX")
    C.check(layer.weight.grad.float().cpu().numpy(), r["dW"], "dW")
    sig = 1.0 / (1.0 + np.exp(-layer.raw.detach().double().cpu().numpy()))
    graw = layer.raw.grad.double().cpu().numpy()
    assert graw[0] == 0.0
    bp, bn = grads_bound(dys, xs, r["q"], M)
    assert abs(graw[1] - r["g_wp"] * sig[1]) <= (bp + 1e-6 * abs(r["g_wp"])) * sig[1] + 1e-6 * abs(graw[1])
    assert abs(graw[2] - r["g_wn"] * sig[2]) <= (bn + 1e-6 * abs(r["g_wn"])) * sig[2] + 1e-6 * abs(graw[2])
    codes, params = layer.export_inference()
    assert np.array_equal(codes.cpu().numpy(), O.pack_codes(O.ttq_codes(w, np.float32(p[0]))))


@pytest.mark.parametrize("M,K,N,split", [
    (300, 1000, 776, 13),      # split tiles forced, dX and dW one after the other
    (2048, 1024, 1024, None),  # dX and dW in one paired launch, both split
])
def test_ttq_graph_replays_match_eager(M, K, N, split, set_knobs):
    """ttq_quantize, ttq_fwd and ttq_bwd (with the scale gradients) captured
    once into a HIP graph and replayed three times, with eager calls on the
    same workspace between the replays: every replay writes the eager
    outputs bit for bit (split-tile counters are left cleared by every
    launch; the gradient partials are rewritten in full by every call)."""
    if split is not None:
        set_knobs(split_ctas=split)
    from ternary_weight_quantization_amd import binding as B
    from tests.gpu_util import dev_bf16
    inp = WL.custom_inputs(M, K, N, seed=M + N + 1)
    note(f"ttq graph replays M={M} K={K} N={N} split={split}")
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    W, x, dY = dev_bf16(inp["W"]), dev_bf16(inp["x"]), dev_bf16(inp["dY"])
    params = torch.empty((3,), dtype=torch.float32, device=dev)
    B.ttq_init(W, params, torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev))
    t = dict(codes=torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev),
             wt=torch.empty((N, Kp), dtype=torch.bfloat16, device=dev),
             y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
             dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
             dW=torch.empty((N, K), dtype=torch.bfloat16, device=dev),
             grads=torch.empty((2,), dtype=torch.float32, device=dev))
    ws = torch.empty((max(B.ttq_workspace_bytes(M, N, K), 256),), dtype=torch.uint8, device=dev)

    def step():
        B.ttq_quantize(W, params, t["codes"], t["wt"])
        B.ttq_fwd(x, t["wt"], t["y"], workspace=ws)
        B.ttq_bwd(dY, x, t["wt"], t["codes"], K, dX=t["dX"], dW=t["dW"], grads=t["grads"], workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in t.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for v in t.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k, v in t.items():
            assert torch.equal(v, ref[k]), (r, k)
        step()
        torch.cuda.synchronize()
        for k in ("y", "dX", "dW", "grads"):
            assert torch.equal(t[k], ref[k]), ("eager", r, k)


def _codes_case(M, K, N, seed, params=None):
    """Inputs, codes and params on the GPU for a ttq_fwd_codes case."""
    from ternary_weight_quantization_amd import binding as B
    from tests.gpu_util import dev_bf16, dev_weight
    inp = WL.custom_inputs(M, K, N, seed=seed)
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    W = dev_weight(inp["W"])
    if params is None:
        p = torch.empty((3,), dtype=torch.float32, device=dev)
        B.ttq_init(W, p, torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev))
    else:
        p = torch.tensor(np.asarray(params, dtype=np.float32), device=dev)
    codes = torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev)
    wt = torch.empty((N, Kp), dtype=torch.bfloat16, device=dev)
    B.ttq_quantize(W, p, codes, wt)
    return inp, dev_bf16(inp["x"]), codes, wt, p


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 32), (5, 512, 200), (32, 2560, 6912), (33, 640, 96), (64, 6912, 2560), (17, 1000, 77),
])
def test_ttq_fwd_codes_few_tokens(M, K, N):
    """ttq_fwd_codes at M <= 64 (the few-token kernel reading the 2-bit codes
    once; K % 8 == 0, K = 1000 with a partial last chunk) against the
    oracle's forward on the values of the same codes; asymmetric
    parameters."""
    from ternary_weight_quantization_amd import binding as B
    note(f"ttq_fwd_codes few tokens M={M} K={K} N={N}")
    inp0 = WL.custom_inputs(M, K, N, seed=M + K)
    e = float(np.mean(np.abs(w_values(inp0["W"]))))
    params = (np.float32(0.6 * e), np.float32(1.3 * e), np.float32(0.7 * e))
    inp, x, codes, wt, p = _codes_case(M, K, N, seed=M + K, params=params)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.ttq_fwd_codes(x, codes, p, y)
    torch.cuda.synchronize()
    w = w_values(inp["W"])
    q = O.ttq_codes(w, params[0])
    assert np.array_equal(codes.cpu().numpy(), O.pack_codes(q))
    ref = O.ttq_forward(bf(inp["x"]), O.ttq_values(q, params[1], params[2]))
    from tests.gpu_util import host_bf16_bits
    m = C.check(bf(host_bf16_bits(y)), ref, "y_ttq")
    print(f"[ttq codes] M={M} K={K} N={N}: max_rel {m['max_rel']:.2e} norm {m['normwise']:.2e}", flush=True)


@pytest.mark.parametrize("M,K,N,knob", [
    (300, 512, 200, None),    # the GEMM route: codes expanded, then the bf16 GEMM
    (48, 1001, 130, None),    # K % 8 != 0: the GEMM route at few tokens
    (40, 512, 264, "1"),      # the no_skinny knob forces the GEMM route
])
def test_ttq_fwd_codes_gemm_route_matches_ttq_fwd(M, K, N, knob, set_knobs):
    """Through the expanded weight, ttq_fwd_codes gives ttq_fwd's bits on
    ttq_quantize's wt (the same GEMM on the same values)."""
    if knob is not None:
        set_knobs(no_skinny=int(knob))
    from ternary_weight_quantization_amd import binding as B
    from tests.gpu_util import host_bf16_bits
    note(f"ttq_fwd_codes GEMM route M={M} K={K} N={N} knob={knob}")
    inp, x, codes, wt, p = _codes_case(M, K, N, seed=7 * M + N)
    assert B.ttq_fwd_codes_workspace_bytes(M, N, K) > 0
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.ttq_fwd_codes(x, codes, p, y1)
    B.ttq_fwd(x, wt, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    w = w_values(inp["W"])
    delta, wp, wn = (np.float32(v) for v in p.cpu().numpy())
    q = O.ttq_codes(w, delta)
    C.check(bf(host_bf16_bits(y1)), O.ttq_forward(bf(inp["x"]), O.ttq_values(q, wp, wn)), "y_ttq")


def test_ttq_export_and_forward_codes():
    """TTQLinear.export_inference + ttq_forward_codes (the inference route
    from the 2-bit state) against the module's own forward, for a decode
    batch (few-token kernel) and a prefill batch (GEMM route)."""
    from ternary_weight_quantization_amd.ttq_layer import TTQLinear, ttq_forward_codes
    torch.manual_seed(1)
    layer = TTQLinear(512, 384)
    codes, params = layer.export_inference()
    note("ttq export + forward from codes")
    for M in (8, 200):
        x = torch.randn(M, 512, device="cuda").to(torch.bfloat16)
        with torch.no_grad():
            y_ref = layer(x)
        y = ttq_forward_codes(x, codes, params)
        torch.cuda.synchronize()
        C.check(y.float().cpu().numpy(), y_ref.float().cpu().numpy().astype(np.float64), "y_ttq")
        if M == 200:  # the same GEMM on the same values
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
