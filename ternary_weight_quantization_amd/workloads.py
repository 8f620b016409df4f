"""Seeded synthetic inputs for the BitLinear layer.

This module only draws random numbers and rounds them to the input dtypes
(bf16 as uint16 bit patterns, or float32). It holds none of the layer's
arithmetic, so the CPU oracle and the HIP path can both be fed from it.

Workloads follow the shapes and distributions of the layers the pages time
("bitnet-qat-train", Usage and Measured behavior: a 2560 -> 6912 layer at
batch 8x512 with bf16 master weights, and an 8-layer 2560 <-> 6912 stack at
batch 4x512); weights use the kaiming-uniform(a=sqrt(5)) bound 1/sqrt(fan_in)
of "bitlinear.py" ``BitLinear.__init__``. Draw order is x, W, dY from one
``numpy.random.Generator(PCG64(seed))``; draws are float32 and are rounded to
bf16 with round-half-to-even.
"""

import math

import numpy as np

CONFIGS = {
    # name: (M, K, N, w_dtype, kind)
    "c1_small": dict(M=64, K=256, N=128, w_dtype="f32", kind="small"),
    "c2_up_4096x2560x6912": dict(M=4096, K=2560, N=6912, w_dtype="bf16", kind="kaiming"),
    "c3_down_4096x6912x2560": dict(M=4096, K=6912, N=2560, w_dtype="bf16", kind="kaiming"),
    "c5_skinny_32x6912x2560": dict(M=32, K=6912, N=2560, w_dtype="bf16", kind="outlier"),
}

# 8-layer stack, alternating up (2560 -> 6912) and down (6912 -> 2560),
# batch 4x512 tokens.
STACK = dict(M=2048, dims=[2560, 6912] * 4 + [2560], w_dtype="bf16")


def f32_to_bf16_bits(a):
    """float32 -> bf16 bit patterns (uint16), round half to even.
    Inputs are finite draws; no NaN handling."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    # finite inputs: u + 0x8000 stays below 2^32
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _uniform(rng, shape, bound):
    u = rng.random(shape, dtype=np.float32)
    return ((u * np.float32(2.0) - np.float32(1.0)) * np.float32(bound)).astype(np.float32)


def layer_inputs(name, seed=0):
    """Inputs of one named layer workload: dict with
    x (uint16 bf16 bits [M, K]), W (uint16 bf16 bits or float32 [N, K]),
    dY (uint16 bf16 bits [M, N]) and the sizes."""
    c = CONFIGS[name]
    M, K, N = c["M"], c["K"], c["N"]
    rng = np.random.Generator(np.random.PCG64(seed))
    if c["kind"] == "small":
        x = _normal(rng, (M, K))
        w = _uniform(rng, (N, K), 1.0 / 16.0)
        dy = _normal(rng, (M, N))
    elif c["kind"] == "kaiming":
        x = _normal(rng, (M, K))
        w = _uniform(rng, (N, K), 1.0 / math.sqrt(K))
        dy = _normal(rng, (M, N))
    elif c["kind"] == "outlier":
        # Student-t(3) activations, 1% of the channels scaled x20;
        # N(0, 0.02) weights with exactly 10% of the entries set to 0.
        x = rng.standard_t(3, size=(M, K)).astype(np.float32)
        n_out = int(round(0.01 * K))
        chans = rng.choice(K, size=n_out, replace=False)
        x[:, chans] *= np.float32(20.0)
        w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        n_zero = int(round(0.1 * N * K))
        zidx = rng.choice(N * K, size=n_zero, replace=False)
        w.reshape(-1)[zidx] = np.float32(0.0)
        dy = _normal(rng, (M, N))
    else:
        raise KeyError(c["kind"])
    W = w if c["w_dtype"] == "f32" else f32_to_bf16_bits(w)
    return dict(name=name, M=M, K=K, N=N, w_dtype=c["w_dtype"],
                x=f32_to_bf16_bits(x), W=W, dY=f32_to_bf16_bits(dy))


def stack_inputs(seed=0, M=None, dims=None):
    """Inputs of the 8-layer stack: x [M, dims[0]], W_i [dims[i+1], dims[i]],
    dY [M, dims[-1]] (all bf16 bits). Draw order x, W_0..W_7, dY."""
    M = STACK["M"] if M is None else M
    dims = STACK["dims"] if dims is None else dims
    rng = np.random.Generator(np.random.PCG64(seed))
    x = f32_to_bf16_bits(_normal(rng, (M, dims[0])))
    Ws = []
    for i in range(len(dims) - 1):
        fan_in, fan_out = dims[i], dims[i + 1]
        Ws.append(f32_to_bf16_bits(_uniform(rng, (fan_out, fan_in), 1.0 / math.sqrt(fan_in))))
    dY = f32_to_bf16_bits(_normal(rng, (M, dims[-1])))
    return dict(M=M, dims=list(dims), x=x, Ws=Ws, dY=dY)


def custom_inputs(M, K, N, seed=0, w_dtype="bf16", w_bound=None):
    """A layer of arbitrary size with the kaiming recipe (used for ragged and
    edge shapes): x, dY ~ N(0, 1), W ~ U(+-bound), bound = 1/sqrt(K) unless
    given."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (M, K))
    bound = (1.0 / math.sqrt(max(K, 1))) if w_bound is None else w_bound
    w = _uniform(rng, (N, K), bound)
    dy = _normal(rng, (M, N))
    W = w if w_dtype == "f32" else f32_to_bf16_bits(w)
    return dict(name=f"custom_{M}x{K}x{N}", M=M, K=K, N=N, w_dtype=w_dtype,
                x=f32_to_bf16_bits(x), W=W, dY=f32_to_bf16_bits(dy))


def tiny_net_inputs():
    """The 3-layer 7 -> 6 -> 5 -> 4 net of "1BitTraining.md" at batch 2:
    legacy ``np.random.seed(0)`` draws in the script's order (W1, W2, W3,
    x0, target), float64."""
    state = np.random.RandomState(0)
    W1 = state.randn(6, 7)
    W2 = state.randn(5, 6)
    W3 = state.randn(4, 5)
    x0 = state.randn(2, 7)
    target = state.randn(2, 4)
    return dict(Ws=[W1, W2, W3], x0=x0, target=target)
