"""bitnet_quantize_static (the allocation-free variant of bitnet_quantize,
its scratch in a device array of the library) against bitnet_quantize with a
caller workspace, through the C ABI: bit for bit on two calls in a row, the
second with a smaller input, so that the second also shows that nothing the
first left in the shared array leaks into its results."""

import numpy as np
import pytest
import torch

from ternary_weight_quantization_amd import workloads as WL

pytestmark = pytest.mark.gpu


def _run(B, inp, static):
    from tests.gpu_util import dev_bf16, dev_weight
    M, K, N = inp["M"], inp["K"], inp["N"]
    Kp = B.bitnet_k_pad(K)
    dev = torch.device("cuda")
    W, x = dev_weight(inp["W"]), dev_bf16(inp["x"])
    t = dict(w_packed=torch.full((N, Kp // 4), 0x55, dtype=torch.uint8, device=dev),
             gamma=torch.full((1,), -1.0, dtype=torch.float32, device=dev),
             x_q=torch.full((M, Kp), 99, dtype=torch.int8, device=dev),
             s_x=torch.full((M,), -1.0, dtype=torch.float32, device=dev))
    if static:
        B.bitnet_quantize_static(W, x, t["w_packed"], t["gamma"], t["x_q"], t["s_x"])
    else:
        ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
        B.bitnet_quantize(W, x, t["w_packed"], t["gamma"], t["x_q"], t["s_x"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in t.items()}


def test_quantize_static_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from ternary_weight_quantization_amd import binding as B
    from tests.gpu_util import note
    for M, K, N, wd in ((4096, 2560, 6912, "bf16"), (40, 1000, 300, "f32")):
        inp = WL.custom_inputs(M, K, N, seed=M + N, w_dtype=wd)
        note(f"quantize static M={M} K={K} N={N} W={wd}")
        got = _run(B, inp, True)
        ref = _run(B, inp, False)
        for k in ref:
            assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), (M, K, N, k)
