"""GPU tests of the one-pass weight quantization (bitnet_quantize and
bitnet_ternarize_pack for bf16 weights with K % 64 == 0): W is read once
and held in registers while the workgroups exchange their absmean partials
through tagged records in the workspace. Checked bit for bit against the
oracle (gamma, packed codes, x_q, s), under a forced give-up of every wait
(each workgroup then computes the missing partials itself), across graph
replays whose weight changes between replays (a replay must not accept the
previous replay's records), and from a workspace holding arbitrary bytes."""

import numpy as np
import pytest
import torch

import oracle as O
from ternary_weight_quantization_amd import binding as B
from ternary_weight_quantization_amd import workloads as WL
from tests.gpu_util import dev_bf16, dev_weight, knobs, note, w_values

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bufs(M, N, Kp, dev):
    return dict(w_packed=torch.full((N, Kp // 4), 0x55, dtype=torch.uint8, device=dev),
                gamma=torch.full((1,), -1.0, dtype=torch.float32, device=dev),
                x_q=torch.full((M, Kp), 99, dtype=torch.int8, device=dev),
                s_x=torch.full((M,), -1.0, dtype=torch.float32, device=dev))


def _host(t):
    return {k: v.cpu().numpy() for k, v in t.items()}


def _check_oracle(out, W_bits, x_bits, Kp):
    w = w_values(W_bits)
    g = O.absmean_gamma(w)
    assert np.float32(out["gamma"][0]).view(np.uint32) == np.float32(g).view(np.uint32)
    assert np.array_equal(out["w_packed"], O.pack_codes(O.ternary_codes(w, g), Kp))
    if x_bits is not None:
        x_q, s = O.act_quant(WL.bf16_bits_to_f32(x_bits).astype(np.float64), Kp)
        assert np.array_equal(out["x_q"], x_q)
        assert np.array_equal(out["s_x"].view(np.uint32), s.view(np.uint32))


def _ws(N, K, dev, fill=None):
    n = B.bitnet_ternarize_workspace_bytes(N, K)
    if fill is None:
        return torch.empty((n,), dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(fill)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)


def _pub_words(ws):
    """The 256 publication words of the one-pass records (after the 256
    fp64 partials of the two-pass kernels; records are 16 bytes: partial,
    then word)."""
    return ws.cpu().numpy()[2048:2048 + 256 * 16].view(np.uint64)[1::2]


def _assert_in_step(ws, seq=None):
    """Every record holds the same word after a launch (each block wrote its
    own once); with `seq`, that word's launch sequence number."""
    w = _pub_words(ws)
    assert np.all(w == w[0]), np.unique(w)
    if seq is not None:
        assert int(w[0]) & 0xFFFF == seq


SHAPES = [
    (4096, 2560, 6912),  # the up-projection: 17 vectors per thread, 64 threads x 5 chunks per row
    (4096, 6912, 2560),  # the down-projection: 128 threads x 7 chunks per row
    (64, 256, 128),      # few vectors: most threads hold none
    (3, 512, 200),       # ragged N and M, rows of 64 threads x 1 chunk
    (17, 3072, 8100),    # 24.9 M weights: 24 vectors per thread
    (1, 7168, 96),       # the longest rows that share the launch (128 threads x 7 chunks)
    (1, 64, 1),          # one code row of four words, one activation row: a single block holds data
    (2, 128, 3),         # a handful of vectors over the 131072 threads
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_onepass_matches_oracle(M, K, N):
    """bitnet_quantize and bitnet_ternarize_pack + bitnet_act_quant on shapes
    the one-pass kernel takes: every output bit equals the oracle's, and
    every record holds the launch's word afterwards."""
    inp = WL.custom_inputs(M, K, N, seed=7 * M + K, w_dtype="bf16")
    note(f"one-pass quantize M={M} K={K} N={N}")
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    assert Kp == K
    W, x = dev_weight(inp["W"]), dev_bf16(inp["x"])
    ws = _ws(N, K, dev)
    fused = _bufs(M, N, Kp, dev)
    B.bitnet_quantize(W, x, fused["w_packed"], fused["gamma"], fused["x_q"], fused["s_x"], ws)
    torch.cuda.synchronize()
    _assert_in_step(ws, 1)
    sep = _bufs(M, N, Kp, dev)
    B.bitnet_ternarize_pack(W, sep["w_packed"], sep["gamma"], ws)
    B.bitnet_act_quant(x, sep["x_q"], sep["s_x"])
    torch.cuda.synchronize()
    _assert_in_step(ws, 1)
    a, b = _host(fused), _host(sep)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    _check_oracle(a, inp["W"], inp["x"], Kp)


@pytest.mark.parametrize("M,K,N", [(4096, 2560, 6912), (64, 256, 128)])
def test_onepass_waits_given_up(M, K, N):
    """With a spin limit of 0 every workgroup looks at each record once and
    computes every partial not yet published itself (counted): the same
    bits. With the default limit no partial is recomputed."""
    inp = WL.custom_inputs(M, K, N, seed=11 * M + K, w_dtype="bf16")
    note(f"one-pass quantize, waits given up, M={M} K={K} N={N}")
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    W, x = dev_weight(inp["W"]), dev_bf16(inp["x"])
    ws = _ws(N, K, dev)
    ref = _bufs(M, N, Kp, dev)
    B.bitnet_quantize_recomputes()
    B.bitnet_quantize(W, x, ref["w_packed"], ref["gamma"], ref["x_q"], ref["s_x"], ws)
    assert B.bitnet_quantize_recomputes() == 0  # every block resident: no wait gave up
    forced, alone = _bufs(M, N, Kp, dev), _bufs(M, N, Kp, dev)
    with knobs(spin_limit=0):
        B.bitnet_quantize(W, x, forced["w_packed"], forced["gamma"], forced["x_q"], forced["s_x"], ws)
        B.bitnet_ternarize_pack(W, alone["w_packed"], alone["gamma"], ws)
    n_re = B.bitnet_quantize_recomputes()  # synchronizes
    if N * K >= 1 << 20:  # blocks publish microseconds apart: some record is missed
        assert n_re > 0
    _assert_in_step(ws, 1)
    a, b, c = _host(ref), _host(forced), _host(alone)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    for k in ("w_packed", "gamma"):
        assert np.array_equal(a[k].view(np.uint8), c[k].view(np.uint8)), k
    _check_oracle(a, inp["W"], inp["x"], Kp)


@pytest.mark.parametrize("M,K,N", [(4096, 2560, 6912), (64, 256, 128)])
def test_onepass_graph_replays_with_changing_weight(M, K, N):
    """A captured bitnet_quantize replayed four times, the weight and the
    activations rewritten in place (eagerly) before each replay: every
    replay gives the bits of an eager call on the same values. A replay
    reuses the captured tag, so a replay that accepted the previous replay's
    publication words would read the previous weight's partials; the words'
    sequence numbers (1, 2, 3, 4 here) keep them apart."""
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    inps = [WL.custom_inputs(M, K, N, seed=100 + r, w_dtype="bf16") for r in range(4)]
    W = dev_weight(inps[0]["W"]).clone()
    x = dev_bf16(inps[0]["x"]).clone()
    ws = _ws(N, K, dev)
    out = _bufs(M, N, Kp, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the binding on the capture stream
        B.bitnet_quantize(W, x, out["w_packed"], out["gamma"], out["x_q"], out["s_x"], ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.bitnet_quantize(W, x, out["w_packed"], out["gamma"], out["x_q"], out["s_x"], ws)
    ws_e = _ws(N, K, dev)
    for r, inp in enumerate(inps):
        note(f"one-pass quantize graph replay {r} M={M} K={K} N={N}")
        W.copy_(dev_weight(inp["W"]))
        x.copy_(dev_bf16(inp["x"]))
        g.replay()
        torch.cuda.synchronize()
        eager = _bufs(M, N, Kp, dev)
        B.bitnet_quantize(W, x, eager["w_packed"], eager["gamma"], eager["x_q"], eager["s_x"], ws_e)
        torch.cuda.synchronize()
        a, b = _host(out), _host(eager)
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (r, k)
        _assert_in_step(ws, r + 1)  # the replays' sequence: 1, 2, 3, 4
        if r in (0, 3):
            _check_oracle(a, inp["W"], inp["x"], Kp)
    del g


def test_onepass_workspace_with_arbitrary_bytes():
    """A workspace full of random bytes: the tags of this launch match none
    of its words."""
    M, K, N = 256, 2560, 6912
    inp = WL.custom_inputs(M, K, N, seed=5, w_dtype="bf16")
    note(f"one-pass quantize, random workspace bytes, M={M} K={K} N={N}")
    dev = torch.device("cuda")
    Kp = B.bitnet_k_pad(K)
    W, x = dev_weight(inp["W"]), dev_bf16(inp["x"])
    for seed in (1, 2):
        ws = _ws(N, K, dev, fill=seed)
        t = _bufs(M, N, Kp, dev)
        B.bitnet_quantize(W, x, t["w_packed"], t["gamma"], t["x_q"], t["s_x"], ws)
        torch.cuda.synchronize()
        _check_oracle(_host(t), inp["W"], inp["x"], Kp)
        _assert_in_step(ws, 1)
