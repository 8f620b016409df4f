"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: gamma, ternary codes / packed bytes, int8 activations, their
scales and the INT32 accumulators. Within tolerance (max relative error
<= 8e-3 with the floors of ``oracle.compare``, normwise <= 5e-3): y, dX, dW.
References are built from the same inputs by the oracle; where the GPU
chains layers, each layer is checked on the GPU's own input.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import compare as C
from ternary_weight_quantization_amd import workloads as WL
from tests.gpu_util import note, run_layer, w_values, dev_bf16, host_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from ternary_weight_quantization_amd import binding
    binding.lib()


def bf(bits):
    return WL.bf16_bits_to_f32(bits).astype(np.float64)


def check_layer(inp, g, x_bits=None, full=True, n_samples=20000, seed=0):
    """Compare one layer's GPU outputs `g` with the oracle. Returns metrics."""
    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = O.k_pad(K)
    w = w_values(inp["W"])
    x = bf(inp["x"] if x_bits is None else x_bits)
    dY = bf(inp["dY"])
    gamma = O.absmean_gamma(w)
    assert np.float32(g["gamma"]).view(np.uint32) == np.float32(gamma).view(np.uint32), (g["gamma"], gamma)
    q = O.ternary_codes(w, gamma)
    assert np.array_equal(g["packed"], O.pack_codes(q, Kp))
    x_q, s = O.act_quant(x, Kp)
    assert np.array_equal(g["s"].view(np.uint32), s.view(np.uint32))
    assert np.array_equal(g["x_q"], x_q)
    y_gpu = bf(g["y_bits"])
    out = dict(near_w=C.near_boundary_weights(w, gamma), near_x=C.near_boundary_acts(x, s))
    if full:
        acc = O.forward_acc(x_q, q)
        if "acc" in g:
            assert np.array_equal(g["acc"], acc)
        out["y"] = C.check(y_gpu, O.forward_y(acc, s, gamma), "y")
        if "dX" in g or "dW" in g:
            dX_ref, dW_ref = O.backward(dY, x_q, s, q, gamma)
            if "dX" in g:
                out["dX"] = C.check(g["dX"], dX_ref, "dX")
            if "dW" in g:
                out["dW"] = C.check(g["dW"], dW_ref, "dW")
    else:
        rng = np.random.default_rng(seed)
        r = rng.integers(0, M, n_samples)
        c = rng.integers(0, N, n_samples)
        if "acc" in g:
            assert np.array_equal(g["acc"][r, c], O.acc_elements(x_q, q, r, c))
        out["y"] = C.check(y_gpu[r, c], O.y_elements(x_q, s, q, gamma, r, c), "y")
        if "dX" in g:
            rk = rng.integers(0, K, n_samples)
            ref = O.dx_elements(dY, q, gamma, r, rk)
            # the floor uses the RMS of the sampled reference
            out["dX"] = C.check(g["dX"][r, rk], ref, "dX")
        if "dW" in g:
            rn = rng.integers(0, N, n_samples)
            rk = rng.integers(0, K, n_samples)
            out["dW"] = C.check(g["dW"][rn, rk], O.dw_elements(dY, x_q, s, rn, rk), "dW")
    print(f"[parity] {inp.get('name', '')}: " + ", ".join(
        f"{k}=max_rel {v['max_rel']:.2e} norm {v['normwise']:.2e}" if isinstance(v, dict) else f"{k}={v}"
        for k, v in out.items()), flush=True)
    return out


@pytest.mark.parametrize("name", list(WL.CONFIGS))
def test_config_full_parity(name):
    inp = WL.layer_inputs(name, seed=0)
    note(f"config {name} M={inp['M']} K={inp['K']} N={inp['N']} W={inp['w_dtype']}")
    g = run_layer(inp)
    check_layer(inp, g, full=True)


@pytest.mark.parametrize("M,K,N,wd", [
    (1, 1, 1, "bf16"),
    (2, 7, 6, "f32"),
    (3, 64, 5, "bf16"),
    (257, 320, 200, "bf16"),
    (300, 1000, 777, "bf16"),
    (520, 1001, 263, "f32"),
    (33, 130, 513, "bf16"),
    (1024, 520, 96, "bf16"),
    (96, 2048, 1030, "f32"),
])
def test_ragged_shapes(M, K, N, wd):
    inp = WL.custom_inputs(M, K, N, seed=M + K + N, w_dtype=wd)
    note(f"ragged M={M} K={K} N={N} W={wd}")
    g = run_layer(inp)
    check_layer(inp, g, full=True)


def test_edge_all_zero_weight():
    inp = WL.custom_inputs(64, 192, 96, seed=5)
    inp["W"] = np.zeros_like(inp["W"])
    note("edge: all-zero W")
    g = run_layer(inp)
    assert g["gamma"] == np.float32(1e-8)
    assert np.all(g["packed"] == 0)
    assert np.all(g["y_bits"] == 0) and np.all(g["dX"] == 0)
    check_layer(inp, g)


def test_edge_zero_rows_and_ties():
    inp = WL.custom_inputs(70, 256, 80, seed=6)
    x = inp["x"].copy()
    x[3] = 0                          # an all-zero row
    # a row whose absmax has significand 254/128: (2j+1)/128 give 127x/s = j + 1/2
    x[5] = 0
    x[5, 0] = WL.f32_to_bf16_bits(np.array([254.0 / 128.0], np.float32))[0]
    for j in range(1, 100):
        x[5, j] = WL.f32_to_bf16_bits(np.array([(2 * j + 1) / 128.0 * (1 if j % 2 else -1)], np.float32))[0]
    x[6] = 0
    x[6, 0] = WL.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
    x[6, 1] = WL.f32_to_bf16_bits(np.array([1.5], np.float32))[0]  # x = s/2 -> 63.5 -> 64
    inp["x"] = x
    # weights: a pattern with mean |w| = 1 and exact ties at +-gamma/2
    w = np.tile(np.array([2.0, 0.5, 1.0, -0.5, 1.5, -1.5, -1.0, 0.0], dtype=np.float32), (80, 32))
    inp["W"] = WL.f32_to_bf16_bits(w)
    note("edge: zero rows and ties")
    g = run_layer(inp)
    assert g["gamma"] == np.float32(1.0)
    assert np.all(g["s"][3] == np.float32(1e-8)) and np.all(g["x_q"][3] == 0)
    assert np.all(bf(g["y_bits"])[3] == 0)
    assert g["x_q"][6, 1] == 64
    assert all(int(g["x_q"][5, j]) % 2 == 0 for j in range(1, 100))
    check_layer(inp, g)


def test_tiny_net_through_the_abi():
    """The 7 -> 6 -> 5 -> 4 net of "1BitTraining.md" at batch 2, every layer
    through the C ABI (float32 masters, bf16 activations, K = 7, 6, 5
    padded to 64). Each layer matches the oracle on its own GPU input, and
    the STE weight gradients have the signs of dL/dQ (torch autograd on the
    CPU with the quantised weights as leaves)."""
    d = WL.tiny_net_inputs()
    Ws = [w.astype(np.float32) for w in d["Ws"]]
    x_bits = WL.f32_to_bf16_bits(d["x0"].astype(np.float32))
    xdev = dev_bf16(x_bits)
    layers = []
    for i, W in enumerate(Ws):
        N, K = W.shape
        inp = dict(name=f"tiny{i}", M=2, K=K, N=N, W=W, x=host_bf16_bits(xdev),
                   dY=np.zeros((2, N), np.uint16))
        note(f"tiny net layer {i} K={K} N={N}")
        g = run_layer(inp, dx=False, dw=False, xdev=xdev)
        check_layer(inp, g)
        layers.append((inp, g))
        xdev = g["y_dev"]
    y = bf(layers[-1][1]["y_bits"])
    dY_bits = WL.f32_to_bf16_bits((y - d["target"]).astype(np.float32))
    grads = [None] * 3
    for i in (2, 1, 0):
        inp, _ = layers[i]
        inp = dict(inp, dY=dY_bits)
        g = run_layer(inp, xdev=dev_bf16(inp["x"]))
        check_layer(inp, g)
        grads[i] = g["dW"]
        dY_bits = WL.f32_to_bf16_bits(g["dX"].astype(np.float32))
    Q = []
    for inp, g in layers:
        w = w_values(inp["W"])
        gm = O.absmean_gamma(w)
        Q.append(torch.tensor(O.w_hat(O.ternary_codes(w, gm), gm), requires_grad=True))
    a = None
    for i, (inp, g) in enumerate(layers):
        K = inp["K"]
        xq, s = O.act_quant(bf(inp["x"]))
        xh = torch.tensor(O.x_hat(xq, s, K))
        a = xh if a is None else a + (xh - a).detach()
        a = a @ Q[i].T
    loss = 0.5 * torch.sum((a - torch.tensor(d["target"])) ** 2)
    loss.backward()
    for i in range(3):
        assert np.array_equal(np.sign(grads[i]), np.sign(Q[i].grad.numpy())), i


@pytest.mark.parametrize("M,K,N,wd,G", [
    (300, 1000, 777, "bf16", 3),      # 2 pieces per tile
    (300, 1000, 777, "bf16", 13),     # 2-3 pieces per tile
    (300, 1000, 777, "bf16", 64),     # fwd: one stage per workgroup, 8 pieces per tile
    (520, 1001, 263, "f32", 5),       # f32 dW, ragged tails
    (1024, 2560, 1536, "bf16", 256),  # a full grid
])
def test_split_tiles_forced(M, K, N, wd, G, set_knobs):
    """Output tiles split over G workgroups (stream-K) on all three GEMMs:
    integer state and accumulators stay bit-exact, the bf16 outputs stay
    within tolerance, and a repeat gives identical bits (the partial tiles
    are added in a fixed order whatever the arrival order)."""
    set_knobs(split_ctas=G)
    inp = WL.custom_inputs(M, K, N, seed=M + K + N + G, w_dtype=wd)
    note(f"split tiles G={G} M={M} K={K} N={N} W={wd}")
    g = run_layer(inp)
    check_layer(inp, g, full=True)
    g2 = run_layer(inp)
    assert np.array_equal(g["acc"], g2["acc"]) and np.array_equal(g["y_bits"], g2["y_bits"])
    assert np.array_equal(g["dX"], g2["dX"]) and np.array_equal(g["dW"], g2["dW"])


def test_split_wait_give_up_is_visible(set_knobs):
    """A wait for another workgroup's partial tile that gives up (forced from
    the host with a zero spin limit, so every kernel still exits normally)
    writes its output tile as NaN and is counted by bitnet_split_timeouts;
    tiles whose partials were all published in time are exact. With the
    default limit the same call is exact again and counts nothing."""
    from ternary_weight_quantization_amd import binding as B
    M, K, N = 1024, 1024, 768
    inp = WL.custom_inputs(M, K, N, seed=77)
    note(f"split wait give-up M={M} K={K} N={N}")
    B.bitnet_split_timeouts()
    set_knobs(split_ctas=64)  # 16 dX tiles of 12 stages: 4 pieces each
    ref = run_layer(inp, acc=False, dw=False)
    assert B.bitnet_split_timeouts() == 0
    set_knobs(split_ctas=64, spin_limit=0)
    g = run_layer(inp, acc=False, dw=False)
    count = B.bitnet_split_timeouts()
    nan_tiles = 0
    for mi in range(0, M, 256):
        for ki in range(0, K, 256):
            t = g["dX"][mi:mi + 256, ki:ki + 256]
            if np.isnan(t).any():
                assert np.isnan(t).all()  # the whole tile, nothing partial
                nan_tiles += 1
            else:
                assert np.array_equal(t, ref["dX"][mi:mi + 256, ki:ki + 256])
    note(f"  timeouts counted {count}, NaN dX tiles {nan_tiles}")
    assert count >= nan_tiles
    set_knobs(split_ctas=64)
    g = run_layer(inp, acc=False, dw=False)
    assert B.bitnet_split_timeouts() == 0
    check_layer(inp, g, full=True)


def test_determinism_repeated_calls():
    inp = WL.custom_inputs(512, 1536, 640, seed=9)
    note("determinism")
    g1 = run_layer(inp)
    g2 = run_layer(inp)
    for k in ("gamma", "packed", "x_q", "s", "acc", "y_bits"):
        assert np.array_equal(np.asarray(g1[k]), np.asarray(g2[k])), k
    assert np.array_equal(g1["dX"], g2["dX"]) and np.array_equal(g1["dW"], g2["dW"])


def test_stack_c4_chain():
    """The 8-layer 2560 <-> 6912 stack at batch 4x512 through QATBitLinear:
    forward chain saving int8 + 2-bit state, then the STE backward chain.
    Only the tensors the checks need are kept (hooks on two activations'
    gradients; nothing retained otherwise). Each checked layer is recomputed
    through the C ABI on the GPU's own input and incoming gradient (bitwise
    equal to the module's results) and compared with the oracle: the first
    (2560 -> 6912) and last (6912 -> 2560) layers in full, accumulators
    included; a middle layer on samples."""
    from ternary_weight_quantization_amd import layer as LY
    d = WL.stack_inputs(seed=0)
    M = d["M"]
    dev = torch.device("cuda")
    layers = [LY.QATBitLinear(d["dims"][i], d["dims"][i + 1], device=dev) for i in range(8)]
    with torch.no_grad():
        for L, Wb in zip(layers, d["Ws"]):
            L.weight.copy_(dev_bf16(Wb))
    torch.cuda.synchronize()
    check = (0, 3, 7)
    acts, grads = {}, {}
    x0 = dev_bf16(d["x"]).requires_grad_(True)
    h = x0
    for i, L in enumerate(layers):
        if i in check:
            acts[i] = h.detach()
        h = L(h)
        if i + 1 in check or i in check:
            acts[i + 1] = h.detach()
            h.register_hook(lambda g, j=i + 1: grads.__setitem__(j, g.detach().clone()))
    note("stack: backward")
    dY = dev_bf16(d["dY"])
    h.backward(dY)
    torch.cuda.synchronize()
    grads[0] = x0.grad
    for i in check:
        L = layers[i]
        K, N = L.in_features, L.out_features
        full = i in (0, 7)
        dy_bits = host_bf16_bits(grads[i + 1]) if i + 1 < 8 else d["dY"]
        inp = dict(name=f"stack{i}", M=M, K=K, N=N, W=d["Ws"][i], x=host_bf16_bits(acts[i]), dY=dy_bits)
        note(f"stack layer {i} ({'full' if full else 'sampled'})")
        g = run_layer(inp, acc=full, xdev=acts[i])
        assert np.array_equal(g["y_bits"], host_bf16_bits(acts[i + 1]))
        assert np.array_equal(g["dW"], bf(host_bf16_bits(L.weight.grad)))
        assert np.array_equal(g["dX"], bf(host_bf16_bits(grads[i])))
        check_layer(inp, g, full=full, seed=i)


@pytest.mark.parametrize("M,K,N", [
    (4096, 6912, 2560),  # the down projection: whole tiles by default (160 tiles, one round)
    (520, 1001, 263),    # ragged
])
def test_forward_bits_independent_of_split(M, K, N, set_knobs):
    """The forward's INT32 sums are exact ("bitnet-qat-train", Semantics), so
    y and the accumulators must not depend on how the output tiles are
    shared out: whole tiles, the cost model's plan and stream-K splits over
    several grids give the same bits; the first is also checked against the
    oracle (sampled at the large shape)."""
    inp = WL.custom_inputs(M, K, N, seed=M + 3 * K + N)
    note(f"forward split invariance M={M} K={K} N={N}")
    set_knobs(split_ctas=-1)
    ref = run_layer(inp, dx=False, dw=False)
    check_layer(inp, ref, full=M * N * K < 5e9)
    for G in (0, 7, 64, 256):
        set_knobs(split_ctas=G)
        g = run_layer(inp, dx=False, dw=False)
        assert np.array_equal(g["acc"], ref["acc"]), G
        assert np.array_equal(g["y_bits"], ref["y_bits"]), G


@pytest.mark.parametrize("M,K,N,split", [
    (300, 1000, 777, 13),     # split tiles in all three GEMMs, separate launches
    (1024, 2560, 1536, None),  # dX and dW in one launch, both split
])
def test_graph_replays_match_eager(M, K, N, split, set_knobs):
    """The four calls captured once into a HIP graph and replayed three
    times, with eager calls on the same workspaces between the replays: each
    replay writes the eager outputs bit for bit (the split-tile counters are
    left cleared by every launch, so a replay with the captured launch tag
    counts its pieces from zero)."""
    if split is not None:
        set_knobs(split_ctas=split)
    inp = WL.custom_inputs(M, K, N, seed=M + N, w_dtype="bf16")
    note(f"graph replays M={M} K={K} N={N} split={split}")
    from ternary_weight_quantization_amd import binding as B
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    W, x, dY = dev_bf16(inp["W"]), dev_bf16(inp["x"]), dev_bf16(inp["dY"])
    t = dict(w_packed=torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev),
             gamma=torch.empty((1,), dtype=torch.float32, device=dev),
             x_q=torch.empty((M, Kp), dtype=torch.int8, device=dev),
             s_x=torch.empty((M,), dtype=torch.float32, device=dev),
             y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
             acc=torch.empty((M, N), dtype=torch.int32, device=dev),
             dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
             dW=torch.empty((N, K), dtype=torch.bfloat16, device=dev))
    ws_t = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    ws_f = torch.empty((max(B.bitlinear_fwd_workspace_bytes(M, N, K), 256),), dtype=torch.uint8, device=dev)
    ws_b = torch.empty((max(B.bitlinear_bwd_workspace_bytes(M, N, K), 256),), dtype=torch.uint8, device=dev)

    def step():
        B.bitnet_ternarize_pack(W, t["w_packed"], t["gamma"], ws_t)
        B.bitnet_act_quant(x, t["x_q"], t["s_x"])
        B.bitlinear_fwd(t["x_q"], t["s_x"], t["w_packed"], t["gamma"], K, t["y"], t["acc"], workspace=ws_f)
        B.bitlinear_bwd(dY, t["x_q"], t["s_x"], t["w_packed"], t["gamma"], K, dX=t["dX"], dW=t["dW"],
                        workspace=ws_b)

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
        step()  # eager calls on the same workspaces between replays
        torch.cuda.synchronize()
        for k in ("y", "dX", "dW"):
            assert torch.equal(t[k], ref[k]), ("eager", r, k)


@pytest.mark.parametrize("M,K,N,with_dx,split", [
    (64, 256, 128, False, None),     # one tile
    (300, 1000, 777, False, None),   # N % 8 != 0: transposing loaders; ragged K
    (520, 1001, 264, True, None),    # with dX in the same call
    (1024, 2560, 1536, True, None),  # dX and dW in one launch, both split
    (300, 1000, 777, False, 13),     # split tiles forced
])
def test_dw_sign1(M, K, N, with_dx, split, set_knobs):
    """dW as 1-bit signs (dW_dtype BITNET_SIGN1). (a) Bit for bit the signs
    of the float32 dW the same call writes with dW_dtype BITNET_F32 (same
    kernels, same summation order), padding bits 0; (b) against the
    oracle's float64 dW at every element whose magnitude exceeds the bound
    M * 2^-24 * sum_m |dY[m,n] * x_hat[m,k]| on the float32 summation error
    (the products are exact), where the sign is fixed whatever the order of
    the sums; elsewhere both bits are signs of an admissible float32 sum;
    (c) a dX computed in the same call is unchanged."""
    if split is not None:
        set_knobs(split_ctas=split)
    inp = WL.custom_inputs(M, K, N, seed=7 * M + N, w_dtype="bf16")
    note(f"dW sign1 M={M} K={K} N={N} dx={with_dx} split={split}")
    from ternary_weight_quantization_amd import binding as B
    dev = torch.device("cuda")
    Kp = O.k_pad(K)
    W, x, dY = dev_bf16(inp["W"]), dev_bf16(inp["x"]), dev_bf16(inp["dY"])
    w_packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev)
    gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    x_q = torch.empty((M, Kp), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    B.bitnet_ternarize_pack(W, w_packed, gamma, ws)
    B.bitnet_act_quant(x, x_q, s_x)
    dX1 = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if with_dx else None
    dX2 = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if with_dx else None
    dWf = torch.empty((N, K), dtype=torch.float32, device=dev)
    bits = torch.full((N, Kp // 8), 0xAB, dtype=torch.uint8, device=dev)
    B.bitlinear_bwd(dY, x_q, s_x, w_packed, gamma, K, dX=dX1, dW=dWf)
    B.bitlinear_bwd(dY, x_q, s_x, w_packed, gamma, K, dX=dX2, dW=bits)
    torch.cuda.synchronize()
    got = bits.cpu().numpy()
    # (a) the signs of the same sums
    assert np.array_equal(got, O.sign1_pack(dWf.cpu().numpy().astype(np.float64), Kp))
    if with_dx:  # (c)
        assert torch.equal(dX1, dX2)
    # (b) the oracle, on its own (bit-exact, checked here) integer state
    w = w_values(inp["W"])
    g = O.absmean_gamma(w)
    q = O.ternary_codes(w, g)
    xq, s = O.act_quant(bf(inp["x"]), Kp)
    assert np.array_equal(w_packed.cpu().numpy(), O.pack_codes(q, Kp))
    assert np.array_equal(x_q.cpu().numpy(), xq)
    dYv = bf(inp["dY"])
    _, dW_ref = O.backward(dYv, xq, s, q, g)
    mag = np.abs(dYv).T @ np.abs(O.x_hat(xq, s, K))
    sure = np.abs(dW_ref) > M * 2.0 ** -24 * mag
    sg, sr = O.sign1_unpack(got, K), O.sign1_unpack(O.sign1_pack(dW_ref, Kp), K)
    assert np.array_equal(sg[sure], sr[sure])
    print(f"[sign1] {M}x{K}x{N}: {int(sure.sum())} of {sure.size} signs fixed by the bound, "
          f"{int(np.sum(sg != sr))} differ elsewhere", flush=True)


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 1),
    (1, 2560, 6912),      # one token
    (17, 1000, 777),      # N % 4 != 0: element stores
    (32, 6912, 2560),     # the skinny workload's shape
    (33, 130, 513),       # two token tiles, ragged
    (64, 6912, 2560),     # the largest M of the few-token path
    (64, 64, 4096),
])
def test_skinny_forward(M, K, N, set_knobs):
    """The few-token forward (M <= 64): y and acc against the oracle (acc
    bit-exact, y within tolerance), and bit for bit the results of the
    large-M GEMM on the same state (forced with the no_skinny knob)."""
    from ternary_weight_quantization_amd import binding as B
    inp = WL.custom_inputs(M, K, N, seed=3 * M + K + N)
    note(f"skinny forward M={M} K={K} N={N}")
    g = run_layer(inp, dx=False, dw=False)
    check_layer(inp, g, full=True)
    dev = torch.device("cuda")
    Kp = O.k_pad(K)
    x_q = torch.from_numpy(g["x_q"]).to(dev)
    s_x = torch.from_numpy(g["s"]).to(dev)
    wp = torch.from_numpy(g["packed"]).to(dev)
    gamma = torch.tensor([g["gamma"]], dtype=torch.float32, device=dev)
    set_knobs(no_skinny=1)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    B.bitlinear_fwd(x_q, s_x, wp, gamma, K, y, acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), g["acc"])
    assert np.array_equal(host_bf16_bits(y), g["y_bits"])
    assert Kp == x_q.shape[1]


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 8),
    (17, 1000, 776),
    (17, 1000, 777),      # N % 8 != 0: the large-M dX
    (32, 6912, 2560),
    (33, 130, 520),
    (64, 2560, 6912),
])
def test_skinny_backward(M, K, N):
    """Few-token backward: dX (the decode-shaped kernel when N % 8 == 0)
    and dW against the oracle, dX alone and with dW in the same call."""
    inp = WL.custom_inputs(M, K, N, seed=5 * M + K + N)
    note(f"skinny backward M={M} K={K} N={N}")
    g = run_layer(inp)
    check_layer(inp, g, full=True)
    g2 = run_layer(inp, dw=False)
    assert np.array_equal(g["dX"], g2["dX"])


@pytest.mark.parametrize("M,K,N,wd", [
    (1, 64, 8, "bf16"),
    (17, 1000, 776, "f32"),    # f32 dW, ragged K (element stores)
    (32, 6912, 2560, "bf16"),
    (33, 130, 520, "bf16"),
    (64, 2560, 6912, "f32"),
])
def test_skinny_dw(M, K, N, wd):
    """Few-token dW (the decode-shaped kernel): against the oracle, alone
    and with dX in the same call."""
    inp = WL.custom_inputs(M, K, N, seed=11 * M + K + N, w_dtype=wd)
    note(f"skinny dW M={M} K={K} N={N} W={wd}")
    g = run_layer(inp, dx=False)
    check_layer(inp, g, full=True)
    g2 = run_layer(inp)
    assert np.array_equal(g["dW"], g2["dW"])


@pytest.mark.parametrize("M,K,N,split", [
    (64, 256, 128, None),     # few tokens
    (17, 1000, 777, None),    # few tokens, N % 4 != 0
    (300, 1000, 777, None),   # large-M GEMM, ragged
    (300, 1000, 777, 7),      # the same, stream-K pieces over 7 workgroups
    (1024, 2560, 1536, None),
])
def test_bias_forward_and_grad(M, K, N, split, set_knobs):
    """Forward with a bias (bitlinear_fwd_bias) and the bias gradient
    (bitlinear_bias_grad): acc bit-exact, y against the oracle's
    forward_y_bias, db (f32 and bf16) against the oracle's exact column
    sums; db bitwise repeatable."""
    from ternary_weight_quantization_amd import binding as B
    if split is not None:
        set_knobs(split_ctas=split)
    inp = WL.custom_inputs(M, K, N, seed=13 * M + N)
    rng = np.random.Generator(np.random.PCG64(M + K + N))
    b_bits = WL.f32_to_bf16_bits(rng.normal(0.0, 0.5, N).astype(np.float32))
    note(f"bias M={M} K={K} N={N} split={split}")
    dev = torch.device("cuda")
    Kp = O.k_pad(K)
    W, x, dY, bias = dev_bf16(inp["W"]), dev_bf16(inp["x"]), dev_bf16(inp["dY"]), dev_bf16(b_bits)
    w_packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev)
    gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    x_q = torch.empty((M, Kp), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    db32 = torch.empty((N,), dtype=torch.float32, device=dev)
    db32b = torch.empty((N,), dtype=torch.float32, device=dev)
    db16 = torch.empty((N,), dtype=torch.bfloat16, device=dev)
    B.bitnet_ternarize_pack(W, w_packed, gamma, ws)
    B.bitnet_act_quant(x, x_q, s_x)
    B.bitlinear_fwd(x_q, s_x, w_packed, gamma, K, y, acc, bias=bias)
    B.bitlinear_bias_grad(dY, db32)
    B.bitlinear_bias_grad(dY, db32b)
    B.bitlinear_bias_grad(dY, db16)
    torch.cuda.synchronize()
    w = w_values(inp["W"])
    g = O.absmean_gamma(w)
    q = O.ternary_codes(w, g)
    xq, s = O.act_quant(bf(inp["x"]), Kp)
    acc_ref = O.forward_acc(xq, q)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    C.check(bf(host_bf16_bits(y)), O.forward_y_bias(acc_ref, s, g, bf(b_bits)), "y_bias")
    db_ref = O.bias_grad(bf(inp["dY"]))
    C.check(db32.cpu().numpy().astype(np.float64), db_ref, "db")
    C.check(bf(host_bf16_bits(db16)), db_ref, "db")
    assert torch.equal(db32, db32b)


def test_layer_with_bias():
    """QATBitLinear(bias=True) through autograd: the bias gradient is the
    library's column sum of the incoming gradient, the output shifts by the
    bias, and from_linear carries a torch Linear's bias."""
    from ternary_weight_quantization_amd import layer as LY
    note("layer with bias")
    torch.manual_seed(0)
    dev = torch.device("cuda")
    lin = torch.nn.Linear(256, 96, bias=True)
    L = LY.QATBitLinear.from_linear(lin.to(dev))
    assert L.bias is not None
    x = torch.randn(4, 8, 256, device=dev).to(torch.bfloat16)
    y = L(x)
    L0 = LY.QATBitLinear.from_linear(torch.nn.Linear(256, 96, bias=False).to(dev))
    with torch.no_grad():
        L0.weight.copy_(L.weight)
    y0 = L0(x)
    with torch.no_grad():
        d = (y.float() - y0.float()) - L.bias.float()
        assert float(d.abs().max()) <= 2.0 ** -7 * float(y.float().abs().max()) + 1e-6
    dy = torch.randn_like(y)
    y.backward(dy)
    ref = O.bias_grad(dy.reshape(-1, 96).float().cpu().numpy().astype(np.float64))
    C.check(L.bias.grad.float().cpu().numpy().astype(np.float64), ref, "db")


@pytest.mark.parametrize("M,K,N,wd", [
    (4096, 2560, 6912, "bf16"),  # the up-projection: 64 threads per row, 8 rows per block
    (300, 6912, 264, "bf16"),    # 128 threads per row
    (64, 256, 128, "f32"),       # f32 masters
    (5, 1000, 33, "bf16"),       # K % 8 != 0: the separate launches
    (3, 9000, 16, "bf16"),       # rows past the shared launch's layout: the separate launches
    (3, 17000, 16, "bf16"),      # rows past the register-resident layout: the separate launches
])
def test_quantize_matches_separate_calls(M, K, N, wd):
    """bitnet_quantize (weight absmean and activation quantization in one
    launch, then the pack) gives the bits of bitnet_ternarize_pack +
    bitnet_act_quant, which the oracle pins."""
    from ternary_weight_quantization_amd import binding as B
    from tests.gpu_util import dev_weight
    inp = WL.custom_inputs(M, K, N, seed=3 * M + K, w_dtype=wd)
    note(f"fused quantize M={M} K={K} N={N} W={wd}")
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    W, x = dev_weight(inp["W"]), dev_bf16(inp["x"])
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    outs = []
    for fused in (True, False):
        t = dict(w_packed=torch.full((N, Kp // 4), 0x55, dtype=torch.uint8, device=dev),
                 gamma=torch.full((1,), -1.0, dtype=torch.float32, device=dev),
                 x_q=torch.full((M, Kp), 99, dtype=torch.int8, device=dev),
                 s_x=torch.full((M,), -1.0, dtype=torch.float32, device=dev))
        if fused:
            B.bitnet_quantize(W, x, t["w_packed"], t["gamma"], t["x_q"], t["s_x"], ws)
        else:
            B.bitnet_ternarize_pack(W, t["w_packed"], t["gamma"], ws)
            B.bitnet_act_quant(x, t["x_q"], t["s_x"])
        torch.cuda.synchronize()
        outs.append({k: v.cpu().numpy() for k, v in t.items()})
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k
    w = w_values(inp["W"])
    g = O.absmean_gamma(w)
    assert np.float32(outs[0]["gamma"][0]).view(np.uint32) == np.float32(g).view(np.uint32)
    assert np.array_equal(outs[0]["w_packed"], O.pack_codes(O.ternary_codes(w, g), Kp))
    x_q, s = O.act_quant(bf(inp["x"]), Kp)
    assert np.array_equal(outs[0]["x_q"], x_q) and np.array_equal(outs[0]["s_x"].view(np.uint32), s.view(np.uint32))
