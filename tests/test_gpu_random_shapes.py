"""Seeded random shapes through the whole BitNet layer and the TTQ layer on
the GPU, each checked against the oracle in full: shapes no fixed case picks
(few or many tokens, K and N ragged or multiples of 8, f32 or bf16 masters),
and so the split, pair and few-token choices they lead to."""

import numpy as np
import pytest
import torch

from ternary_weight_quantization_amd import workloads as WL
from tests.gpu_util import note, run_layer, run_ttq
from tests.test_gpu_parity import check_layer
from tests.test_gpu_ttq import check_ttq

pytestmark = pytest.mark.gpu


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 1600))]))
        K = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 3000)), 8 * int(rng.integers(8, 400))]))
        N = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 3000)), 8 * int(rng.integers(8, 400))]))
        out.append((M, K, N, "f32" if rng.random() < 0.3 else "bf16"))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")


@pytest.mark.parametrize("i,M,K,N,wd", [(i, *s) for i, s in enumerate(_shapes(4242, 16))])
def test_random_shape(i, M, K, N, wd):
    note(f"random shape {i}: M={M} K={K} N={N} W={wd}")
    inp = WL.custom_inputs(M, K, N, seed=5000 + i, w_dtype=wd)
    check_layer(inp, run_layer(inp), full=True)
    check_ttq(inp, run_ttq(inp, dw_f32=(wd == "f32")))


# Shapes on the edges the kernels branch on: the few-token cutoff (M = 64
# runs the decode-shaped kernels, 65 the 256 x 256 tiles), one token more or
# fewer than a whole tile along each output axis, K around the 64-value
# padding and the 128-byte stage, N around the multiple of 8 the 16-byte
# token loads and the paired launch need, and one-row / one-column outputs.
EDGE_SHAPES = [
    (64, 320, 264, "bf16"), (65, 320, 264, "bf16"),
    (64, 129, 255, "f32"), (65, 129, 257, "f32"),
    (255, 64, 256, "bf16"), (257, 65, 256, "bf16"),
    (256, 127, 257, "bf16"), (256, 128, 255, "f32"),
    (513, 256, 511, "bf16"), (511, 257, 513, "bf16"),
    (1, 2560, 6912, "bf16"), (4096, 1, 8, "bf16"), (4096, 8, 1, "bf16"),
    (300, 2560, 8, "bf16"), (300, 8, 2560, "bf16"),
]


@pytest.mark.parametrize("M,K,N,wd", EDGE_SHAPES)
def test_edge_shape(M, K, N, wd):
    note(f"edge shape M={M} K={K} N={N} W={wd}")
    inp = WL.custom_inputs(M, K, N, seed=M * 7 + K * 3 + N, w_dtype=wd)
    check_layer(inp, run_layer(inp), full=True)
