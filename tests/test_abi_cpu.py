"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, answers its size queries, and rejects bad arguments with
the documented codes before touching the GPU (no compute call here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitnet.h")
LIB = os.path.join(ROOT, "ternary_weight_quantization_amd", "libbitnet.so")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EHIP = range(7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:bitnet|bitlinear|ttq)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail("libbitnet.so is not built (run `python -m ternary_weight_quantization_amd.build`)")
    lib = ctypes.CDLL(LIB)
    i64, sz, vp, st = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    lib.bitnet_status_string.restype = ctypes.c_char_p
    lib.bitnet_k_pad.argtypes = [i64]
    lib.bitnet_k_pad.restype = i64
    lib.bitnet_ternarize_workspace_bytes.argtypes = [i64, i64]
    lib.bitnet_ternarize_workspace_bytes.restype = sz
    lib.bitlinear_fwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.bitlinear_fwd_workspace_bytes.restype = sz
    lib.bitlinear_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.bitlinear_bwd_workspace_bytes.restype = sz
    lib.bitnet_ternarize_pack.argtypes = [vp, st, i64, i64, vp, vp, vp, sz, vp]
    lib.bitnet_act_quant.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.bitlinear_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.bitlinear_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, st, vp, sz, vp]
    lib.bitlinear_fwd_bias.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.bitlinear_bias_grad.argtypes = [vp, i64, i64, vp, st, vp]
    lib.ttq_workspace_bytes.argtypes = [i64, i64, i64]
    lib.ttq_workspace_bytes.restype = sz
    lib.ttq_init.argtypes = [vp, st, i64, i64, vp, vp, sz, vp]
    lib.ttq_quantize.argtypes = [vp, st, i64, i64, vp, vp, vp, vp]
    lib.ttq_fwd.argtypes = [vp, vp, i64, i64, i64, vp, vp, sz, vp]
    lib.ttq_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, st, vp, vp, sz, vp]
    lib.ttq_fwd_codes_workspace_bytes.argtypes = [i64, i64, i64]
    lib.ttq_fwd_codes_workspace_bytes.restype = sz
    lib.ttq_fwd_codes.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, sz, vp]
    return lib


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("bitnet_ternarize_pack", "bitnet_act_quant", "bitlinear_fwd", "bitlinear_bwd",
              "bitlinear_fwd_bias", "bitlinear_bias_grad", "ttq_workspace_bytes", "ttq_init", "ttq_quantize",
              "ttq_fwd", "ttq_bwd", "ttq_fwd_codes", "ttq_fwd_codes_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_size_queries(L):
    assert [L.bitnet_k_pad(k) for k in (1, 7, 63, 64, 65, 2560, 6912)] == [64, 64, 64, 64, 128, 2560, 6912]
    assert L.bitnet_k_pad(0) == 0
    assert L.bitnet_ternarize_workspace_bytes(6912, 2560) >= 8 * 256
    # whole output tiles need no workspace; split tiles need tagged counters
    # (16 bytes per tile, rounded to 256) and 256 KiB partial tiles, as many
    # as min(2G, G + T - 1) for G workgroups and T tiles; dW adds its bf16
    # x_hat [M][Kp], dX its fp4 transposed codes [Kp][Np/2]
    assert L.bitlinear_fwd_workspace_bytes(4096, 6912, 2560) == 0
    assert L.bitlinear_fwd_workspace_bytes(64, 128, 256) == 0
    # few tokens (M <= 64): bf16 / f32 dW converts its own x_hat, so both
    # outputs need only dX's fp4 codes [Kp][Np/2]; the size also covers the
    # 1-bit dW output, which runs the large-M route with x_hat [M][Kp]
    assert L.bitlinear_bwd_workspace_bytes(64, 128, 256) == max(2 * 64 * 256, 256 * 128 // 2)
    tile = 64 * 256 * 16
    # at 4096x2560->6912 the two backward products run in one launch: dX
    # stream-K over 15 columns of 8 workgroups (160 tiles on 120: 240
    # slots), dW in whole tiles on the other 136 (no partials); plus the fp4
    # transposed codes [Kp][N/2] and x_hat
    assert L.bitlinear_bwd_workspace_bytes(4096, 6912, 2560) == \
        2560 * 6912 // 2 + 2 * 4096 * 2560 + 2560 + 240 * tile
    # the int8 forward runs whole tiles unless a split saves more than 48
    # stages a piece: 4096x6912->2560 (160 tiles of 54 stages, one round)
    # needs none; one tile of 512 stages splits over 4 workgroups (4 slots)
    assert L.bitlinear_fwd_workspace_bytes(4096, 2560, 6912) == 0
    assert L.bitlinear_fwd_workspace_bytes(256, 256, 65536) == 256 + 4 * tile
    # few tokens: the forward needs none; the backward the larger of the fp4
    # codes [Kp][N/2] (dX, which does not split) and x_hat [M][Kp] (the 1-bit
    # dW route)
    assert L.bitlinear_fwd_workspace_bytes(32, 2560, 6912) == 0
    assert L.bitlinear_bwd_workspace_bytes(32, 2560, 6912) == max(6912 * 2560 // 2, 2 * 32 * 6912)
    assert L.bitlinear_fwd_workspace_bytes(0, 4, 4) == 0
    for code in range(7):
        assert L.bitnet_status_string(code).decode().startswith("BITNET_")


# Fake, never dereferenced device addresses: validation fails before any use.
A = 0x10000000
MISALIGNED = 0x10000008


def test_ternarize_validation(L):
    ws = L.bitnet_ternarize_workspace_bytes(8, 8)
    assert L.bitnet_ternarize_pack(None, 0, 8, 8, A, A, A, ws, None) == ENULL
    assert L.bitnet_ternarize_pack(A, 0, 8, 8, None, A, A, ws, None) == ENULL
    assert L.bitnet_ternarize_pack(A, 0, 8, 8, A, None, A, ws, None) == ENULL
    assert L.bitnet_ternarize_pack(A, 7, 8, 8, A, A, A, ws, None) == EDTYPE
    assert L.bitnet_ternarize_pack(A, 0, 0, 8, A, A, A, ws, None) == ESHAPE
    assert L.bitnet_ternarize_pack(A, 0, 8, -1, A, A, A, ws, None) == ESHAPE
    assert L.bitnet_ternarize_pack(MISALIGNED, 0, 8, 8, A, A, A, ws, None) == EALIGN
    assert L.bitnet_ternarize_pack(A, 0, 8, 8, A, A, None, ws, None) == EWS
    assert L.bitnet_ternarize_pack(A, 0, 8, 8, A, A, A, ws - 1, None) == EWS


def test_act_quant_validation(L):
    assert L.bitnet_act_quant(None, 4, 4, A, A, None) == ENULL
    assert L.bitnet_act_quant(A, 0, 4, A, A, None) == ESHAPE
    assert L.bitnet_act_quant(A, 4, 0, A, A, None) == ESHAPE
    assert L.bitnet_act_quant(A, 4, 4, MISALIGNED, A, None) == EALIGN
    assert L.bitnet_act_quant(A, 4, 4, A, MISALIGNED, None) == EALIGN


def test_fwd_validation(L):
    assert L.bitlinear_fwd(None, A, A, A, 4, 4, 4, A, None, None, 0, None) == ENULL
    assert L.bitlinear_fwd(A, A, A, A, 4, 4, 4, None, None, None, 0, None) == ENULL
    assert L.bitlinear_fwd(A, A, A, A, 0, 4, 4, A, None, None, 0, None) == ESHAPE
    assert L.bitlinear_fwd(A, A, A, A, 4, 4, 1 << 25, A, None, None, 0, None) == ESHAPE
    # operands addressed with 32-bit offsets: (M + 256) * Kp bytes of x_q and
    # (N + 256) * Kp/4 bytes of w_packed must stay within 2^31
    assert L.bitlinear_fwd(A, A, A, A, 1 << 20, 4, 1 << 12, A, None, None, 0, None) == ESHAPE
    assert L.bitlinear_fwd(A, A, A, A, 4, 1 << 22, 1 << 12, A, None, None, 0, None) == ESHAPE
    # the epilogue addresses 32 output rows of N 4-byte values with 32-bit offsets: N <= 2^24
    assert L.bitlinear_fwd(A, A, A, A, 4, (1 << 24) + 64, 64, A, None, None, 0, None) == ESHAPE
    assert L.bitlinear_fwd(A, A, A, A, 4, 4, 4, MISALIGNED, None, None, 0, None) == EALIGN
    assert L.bitlinear_fwd(A, A, A, A, 4, 4, 4, A, MISALIGNED, None, 0, None) == EALIGN
    assert L.bitlinear_fwd(A, A, A, A + 2, 4, 4, 4, A, None, None, 0, None) == EALIGN


def test_gemm_workspace_validation(L):
    need = L.bitlinear_bwd_workspace_bytes(4096, 6912, 2560)
    assert L.bitlinear_bwd(A, A, A, A, A, 4096, 6912, 2560, A, A, 0, A, need - 1, None) == EWS
    assert L.bitlinear_bwd(A, A, A, A, A, 4096, 6912, 2560, A, A, 0, None, need, None) == EWS
    assert L.bitlinear_bwd(A, A, A, A, A, 4096, 6912, 2560, A, A, 0, MISALIGNED + 4, need, None) == EALIGN
    # a forward that splits its one tile (K = 65536) needs split workspace
    need = L.bitlinear_fwd_workspace_bytes(256, 256, 65536)
    assert need > 0
    assert L.bitlinear_fwd(A, A, A, A, 256, 256, 65536, A, None, A, need - 1, None) == EWS


def test_bwd_validation(L):
    assert L.bitlinear_bwd(None, A, A, A, A, 4, 4, 4, A, A, 0, None, 0, None) == ENULL
    assert L.bitlinear_bwd(A, A, A, A, A, 4, 4, 4, None, None, 0, None, 0, None) == ENULL
    assert L.bitlinear_bwd(A, None, A, A, A, 4, 4, 4, None, A, 0, None, 0, None) == ENULL
    assert L.bitlinear_bwd(A, A, A, None, A, 4, 4, 4, A, None, 0, None, 0, None) == ENULL
    assert L.bitlinear_bwd(A, A, A, A, A, 4, 4, 4, None, A, 5, None, 0, None) == EDTYPE
    assert L.bitlinear_bwd(A, A, A, A, A, 4, 0, 4, A, A, 0, None, 0, None) == ESHAPE
    # dY is addressed with 32-bit offsets: (M + 256) * 2N bytes within 2^31
    assert L.bitlinear_bwd(A, A, A, A, A, 1 << 16, 1 << 15, 64, A, None, 0, None, 0, None) == ESHAPE
    assert L.bitlinear_bwd(A, A, A, A, A, 1 << 16, 1 << 15, 64, None, A, 0, None, 0, None) == ESHAPE
    ws = L.bitlinear_bwd_workspace_bytes(4, 4, 4)  # dW's x_hat
    assert L.bitlinear_bwd(MISALIGNED, A, A, A, A, 4, 4, 4, A, A, 0, A, ws, None) == EALIGN
    assert L.bitlinear_bwd(A, A, A, A, A, 4, 4, 4, MISALIGNED, None, 0, A, ws, None) == EALIGN


def test_bias_validation(L):
    # bitlinear_fwd_bias checks what bitlinear_fwd checks, plus the bias alignment
    assert L.bitlinear_fwd_bias(None, A, A, A, A, 4, 4, 4, A, None, None, 0, None) == ENULL
    assert L.bitlinear_fwd_bias(A, A, A, A, A, 0, 4, 4, A, None, None, 0, None) == ESHAPE
    assert L.bitlinear_fwd_bias(A, A, A, A, A + 2, 4, 4, 4, A, None, None, 0, None) == EALIGN
    assert L.bitlinear_bias_grad(None, 4, 4, A, 1, None) == ENULL
    assert L.bitlinear_bias_grad(A, 4, 4, None, 1, None) == ENULL
    assert L.bitlinear_bias_grad(A, 4, 4, A, 2, None) == EDTYPE
    assert L.bitlinear_bias_grad(A, 0, 4, A, 1, None) == ESHAPE
    assert L.bitlinear_bias_grad(A, 4, 4, MISALIGNED, 1, None) == EALIGN


def test_ttq_size_queries(L):
    tile = 64 * 256 * 16
    # no split at a single tile: only the scale-gradient partials (one float2
    # per 128 x 128 tile of dW, rounded up to 256 bytes)
    assert L.ttq_workspace_bytes(64, 128, 256) == 256
    # 4096x2560->6912: dW has 10 x 27 tiles (4 partials each); dX and dW run
    # in one launch planned as the BitNet pair: dX stream-K on 120
    # workgroups (its 160 tiles' counters and 240 partial tiles), dW whole
    partials = (4 * 270 * 8 + 255) // 256 * 256
    assert L.ttq_workspace_bytes(4096, 6912, 2560) == partials + 2560 + 240 * tile
    assert L.ttq_workspace_bytes(0, 4, 4) == 0


def test_ttq_validation(L):
    ws = L.bitnet_ternarize_workspace_bytes(8, 8)
    assert L.ttq_init(None, 0, 8, 8, A, A, ws, None) == ENULL
    assert L.ttq_init(A, 0, 8, 8, None, A, ws, None) == ENULL
    assert L.ttq_init(A, 2, 8, 8, A, A, ws, None) == EDTYPE
    assert L.ttq_init(A, 0, 0, 8, A, A, ws, None) == ESHAPE
    assert L.ttq_init(MISALIGNED, 0, 8, 8, A, A, ws, None) == EALIGN
    assert L.ttq_init(A, 0, 8, 8, A + 2, A, ws, None) == EALIGN
    assert L.ttq_init(A, 0, 8, 8, A, A, ws - 1, None) == EWS
    assert L.ttq_quantize(A, 0, 8, 8, A, None, A, None) == ENULL
    assert L.ttq_quantize(A, 0, 8, 8, A, A, None, None) == ENULL
    assert L.ttq_quantize(A, 1, 8, -8, A, A, A, None) == ESHAPE
    assert L.ttq_quantize(A, 0, 8, 8, A, A, MISALIGNED, None) == EALIGN
    assert L.ttq_fwd(None, A, 4, 4, 4, A, None, 0, None) == ENULL
    assert L.ttq_fwd(A, A, 4, 0, 4, A, None, 0, None) == ESHAPE
    # x is addressed with 32-bit offsets: (M + 256) * 2K bytes within 2^31
    assert L.ttq_fwd(A, A, 1 << 20, 4, 1 << 11, A, None, 0, None) == ESHAPE
    ws = L.ttq_workspace_bytes(4, 4, 4)  # one size for both calls
    assert L.ttq_fwd(A, A, 4, 4, 4, A, None, ws, None) == EWS
    assert L.ttq_fwd(A, A, 4, 4, 4, MISALIGNED, A, ws, None) == EALIGN
    need = L.ttq_workspace_bytes(4096, 6912, 2560)
    assert L.ttq_fwd(A, A, 4096, 6912, 2560, A, A, need - 1, None) == EWS
    ws = L.ttq_workspace_bytes(4, 4, 4)
    assert L.ttq_bwd(A, A, A, A, 4, 4, 4, None, None, 0, None, A, ws, None) == ENULL
    assert L.ttq_bwd(A, A, None, A, 4, 4, 4, A, None, 0, None, A, ws, None) == ENULL
    assert L.ttq_bwd(A, None, A, A, 4, 4, 4, None, A, 0, None, A, ws, None) == ENULL
    # the scale gradients come from dW's epilogue and need the codes
    assert L.ttq_bwd(A, A, A, A, 4, 4, 4, A, None, 0, A, A, ws, None) == ENULL
    assert L.ttq_bwd(A, A, A, None, 4, 4, 4, None, A, 0, A, A, ws, None) == ENULL
    assert L.ttq_bwd(A, A, A, A, 4, 4, 4, None, A, 2, None, A, ws, None) == EDTYPE
    assert L.ttq_bwd(A, A, A, A, 4, 4, 4, None, A, 0, None, A, ws - 1, None) == EWS
    assert L.ttq_bwd(A, A, A, A, 4, 4, 4, None, A, 0, A + 2, A, ws, None) == EALIGN
    assert L.ttq_bwd(A, A, A, A, 4, 4, 4, MISALIGNED, None, 0, None, A, ws, None) == EALIGN


def test_ttq_inverse_softplus_round_trip():
    """TTQLinear keeps its three scalars raw and applies softplus; the raw
    start values are the inverse softplus of the initial (delta, Wp, Wn)
    ("TTQ_VERIFICATION.md", Bugs Fixed item 5). The round trip returns the
    values across the range a layer's E|W| takes (CPU, float64 and the
    float32 the module stores)."""
    import torch
    from ternary_weight_quantization_amd.ttq_layer import _inverse_softplus
    v = torch.tensor([1e-8, 1e-5, 3e-3, 0.02, 0.7, 5.0], dtype=torch.float64)
    r = _inverse_softplus(v)
    assert torch.allclose(torch.nn.functional.softplus(r), v, rtol=1e-12, atol=0)
    r32 = r.float()
    assert torch.allclose(torch.nn.functional.softplus(r32).double(), v, rtol=1e-5, atol=0)


def test_ttq_fwd_codes_size_and_validation(L):
    # few tokens with K % 8 == 0 read the codes directly: no workspace
    assert L.ttq_fwd_codes_workspace_bytes(32, 2560, 6912) == 0
    assert L.ttq_fwd_codes_workspace_bytes(64, 128, 256) == 0
    # otherwise the expanded bf16 weight [N][Kp] (+ the GEMM's split share,
    # none here: whole tiles)
    assert L.ttq_fwd_codes_workspace_bytes(4096, 6912, 2560) == 6912 * 2560 * 2
    assert L.ttq_fwd_codes_workspace_bytes(32, 100, 7) == (100 * 64 * 2 + 255) // 256 * 256
    assert L.ttq_fwd_codes_workspace_bytes(0, 4, 4) == 0
    assert L.ttq_fwd_codes(None, A, A, 4, 4, 8, A, None, 0, None) == ENULL
    assert L.ttq_fwd_codes(A, A, None, 4, 4, 8, A, None, 0, None) == ENULL
    assert L.ttq_fwd_codes(A, A, A, 4, 0, 8, A, None, 0, None) == ESHAPE
    assert L.ttq_fwd_codes(A, A, A, 4, 4, 8, MISALIGNED, None, 0, None) == EALIGN
    assert L.ttq_fwd_codes(A, A, A + 2, 4, 4, 8, A, None, 0, None) == EALIGN
    need = L.ttq_fwd_codes_workspace_bytes(300, 200, 512)
    assert need > 0
    assert L.ttq_fwd_codes(A, A, A, 300, 200, 512, A, None, need, None) == EWS
    assert L.ttq_fwd_codes(A, A, A, 300, 200, 512, A, A, need - 1, None) == EWS
