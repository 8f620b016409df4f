"""ctypes binding of libbitnet.so: the C entry points under the same names.

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks that dtypes, shapes and contiguity match what the C
ABI documents, and passes raw device pointers and the current HIP stream.
All computation happens in the library's kernels. Outputs are preallocated
by the caller, as in the C ABI. If the library is not built this module
raises; there is no other compute path.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitnet.so")

BITNET_OK = 0
BITNET_BF16 = 0
BITNET_F32 = 1
BITNET_SIGN1 = 2

_lib = None


def _hip_runtimes_mapped():
    """Paths of the libamdhip64 copies mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def lib():
    """Load libbitnet.so (after torch, so that both share torch's HIP
    runtime) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m ternary_weight_quantization_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, sz, vp, st = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    L.bitnet_status_string.argtypes = [st]
    L.bitnet_status_string.restype = ctypes.c_char_p
    L.bitnet_k_pad.argtypes = [i64]
    L.bitnet_k_pad.restype = i64
    L.bitnet_ternarize_workspace_bytes.argtypes = [i64, i64]
    L.bitnet_ternarize_workspace_bytes.restype = sz
    L.bitlinear_fwd_workspace_bytes.argtypes = [i64, i64, i64]
    L.bitlinear_fwd_workspace_bytes.restype = sz
    L.bitlinear_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    L.bitlinear_bwd_workspace_bytes.restype = sz
    L.bitnet_ternarize_pack.argtypes = [vp, st, i64, i64, vp, vp, vp, sz, vp]
    L.bitnet_ternarize_pack.restype = st
    L.bitnet_quantize.argtypes = [vp, st, i64, i64, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    L.bitnet_quantize.restype = st
    L.bitnet_quantize_static.argtypes = [vp, st, i64, i64, vp, i64, vp, vp, vp, vp, vp]
    L.bitnet_quantize_static.restype = st
    L.bitnet_code_counts.argtypes = [vp, i64, i64, vp, vp]
    L.bitnet_code_counts.restype = st
    L.bitnet_act_quant.argtypes = [vp, i64, i64, vp, vp, vp]
    L.bitnet_act_quant.restype = st
    L.bitlinear_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    L.bitlinear_fwd.restype = st
    L.bitlinear_fwd_bias.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    L.bitlinear_fwd_bias.restype = st
    L.bitlinear_bias_grad.argtypes = [vp, i64, i64, vp, st, vp]
    L.bitlinear_bias_grad.restype = st
    L.bitlinear_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, st, vp, sz, vp]
    L.bitlinear_bwd.restype = st
    L.ttq_workspace_bytes.argtypes = [i64, i64, i64]
    L.ttq_workspace_bytes.restype = sz
    L.ttq_init.argtypes = [vp, st, i64, i64, vp, vp, sz, vp]
    L.ttq_init.restype = st
    L.ttq_quantize.argtypes = [vp, st, i64, i64, vp, vp, vp, vp]
    L.ttq_quantize.restype = st
    L.ttq_fwd.argtypes = [vp, vp, i64, i64, i64, vp, vp, sz, vp]
    L.ttq_fwd.restype = st
    L.ttq_bwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, st, vp, vp, sz, vp]
    L.ttq_bwd.restype = st
    L.ttq_fwd_codes_workspace_bytes.argtypes = [i64, i64, i64]
    L.ttq_fwd_codes_workspace_bytes.restype = sz
    L.ttq_fwd_codes.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, sz, vp]
    L.ttq_fwd_codes.restype = st
    i32, u32 = ctypes.c_int32, ctypes.c_uint32
    L.bitnet_set_test_knobs.argtypes = [st, st, st, u32]
    L.bitnet_set_test_knobs.restype = None
    L.bitnet_default_spin_limit.argtypes = []
    L.bitnet_default_spin_limit.restype = u32
    L.bitnet_split_timeouts.argtypes = [vp]
    L.bitnet_split_timeouts.restype = st
    L.bitnet_quantize_recomputes.argtypes = [vp]
    L.bitnet_quantize_recomputes.restype = st
    L.bitnet_debug_split_pieces.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64]
    L.bitnet_debug_split_pieces.restype = i64
    L.bitnet_debug_partial_slots.argtypes = [i64, i32]
    L.bitnet_debug_partial_slots.restype = i32
    L.bitnet_debug_mfma_probe.argtypes = [i32, i32, vp, vp, vp]
    L.bitnet_debug_mfma_probe.restype = st
    L.bitnet_debug_cta_order.argtypes = [i32, vp]
    L.bitnet_debug_cta_order.restype = None
    if len(_hip_runtimes_mapped()) > 1:
        raise RuntimeError("more than one libamdhip64 is mapped into this process: "
                           f"{sorted(_hip_runtimes_mapped())}")
    _lib = L
    return _lib


def _check(code):
    if code != BITNET_OK:
        msg = lib().bitnet_status_string(code).decode()
        raise RuntimeError(f"libbitnet: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")


# --- size queries ----------------------------------------------------------

def bitnet_k_pad(K):
    return int(lib().bitnet_k_pad(int(K)))


def bitnet_ternarize_workspace_bytes(N, K):
    return int(lib().bitnet_ternarize_workspace_bytes(int(N), int(K)))


def bitlinear_fwd_workspace_bytes(M, N, K):
    return int(lib().bitlinear_fwd_workspace_bytes(int(M), int(N), int(K)))


def bitlinear_bwd_workspace_bytes(M, N, K):
    return int(lib().bitlinear_bwd_workspace_bytes(int(M), int(N), int(K)))


# --- GEMM workspace ----------------------------------------------------------

_workspaces = {}


def _workspace(nbytes, like, stream):
    """A cached device buffer of at least nbytes for the GEMM calls, one per
    (device, stream): calls on one stream run in order and may share it.
    The library needs no particular contents."""
    if nbytes == 0:
        return None
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    key = (like.device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty((nbytes,), dtype=torch.uint8, device=like.device)
        _workspaces[key] = ws
    return ws


# --- entry points ----------------------------------------------------------

def bitnet_ternarize_pack(W, w_packed, gamma, workspace, stream=None):
    """W [N, K] bf16 or float32 -> w_packed uint8 [N, Kp/4], gamma float32 [1]."""
    N, K = W.shape
    Kp = bitnet_k_pad(K)
    if W.dtype == torch.bfloat16:
        wd = BITNET_BF16
    elif W.dtype == torch.float32:
        wd = BITNET_F32
    else:
        raise TypeError(f"W: expected bfloat16 or float32, got {W.dtype}")
    _need(W, W.dtype, (N, K), "W")
    _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    _need(gamma, torch.float32, (1,), "gamma")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().bitnet_ternarize_pack(_ptr(W), wd, N, K, _ptr(w_packed), _ptr(gamma),
                                       _ptr(workspace), ws_bytes, _stream(stream)))


def bitnet_quantize(W, x, w_packed, gamma, x_q, s_x, workspace, stream=None):
    """bitnet_ternarize_pack(W, ...) and bitnet_act_quant(x, ...) in one call
    (W [N, K] bf16 or float32, x [M, K] bf16)."""
    N, K = W.shape
    M = x.shape[0]
    Kp = bitnet_k_pad(K)
    if W.dtype == torch.bfloat16:
        wd = BITNET_BF16
    elif W.dtype == torch.float32:
        wd = BITNET_F32
    else:
        raise TypeError(f"W: expected bfloat16 or float32, got {W.dtype}")
    _need(W, W.dtype, (N, K), "W")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    _need(gamma, torch.float32, (1,), "gamma")
    _need(x_q, torch.int8, (M, Kp), "x_q")
    _need(s_x, torch.float32, (M,), "s_x")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().bitnet_quantize(_ptr(W), wd, N, K, _ptr(x), M, _ptr(w_packed), _ptr(gamma), _ptr(x_q), _ptr(s_x),
                                 _ptr(workspace), ws_bytes, _stream(stream)))


def bitnet_quantize_static(W, x, w_packed, gamma, x_q, s_x, stream=None):
    """bitnet_quantize with the library's own scratch array: no workspace,
    nothing allocated."""
    N, K = W.shape
    M = x.shape[0]
    Kp = bitnet_k_pad(K)
    if W.dtype == torch.bfloat16:
        wd = BITNET_BF16
    elif W.dtype == torch.float32:
        wd = BITNET_F32
    else:
        raise TypeError(f"W: expected bfloat16 or float32, got {W.dtype}")
    _need(W, W.dtype, (N, K), "W")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    _need(gamma, torch.float32, (1,), "gamma")
    _need(x_q, torch.int8, (M, Kp), "x_q")
    _need(s_x, torch.float32, (M,), "s_x")
    _check(lib().bitnet_quantize_static(_ptr(W), wd, N, K, _ptr(x), M, _ptr(w_packed), _ptr(gamma), _ptr(x_q),
                                        _ptr(s_x), _stream(stream)))


def bitnet_code_counts(w_packed, K, counts, stream=None):
    """counts int64 [2] = (number of -1 codes, number of +1 codes) in
    w_packed uint8 [N, Kp/4] over the true N x K weights."""
    N = w_packed.shape[0]
    _need(w_packed, torch.uint8, (N, bitnet_k_pad(K) // 4), "w_packed")
    _need(counts, torch.int64, (2,), "counts")
    _check(lib().bitnet_code_counts(_ptr(w_packed), N, int(K), _ptr(counts), _stream(stream)))


def bitnet_act_quant(x, x_q, s_x, stream=None):
    """x [M, K] bf16 -> x_q int8 [M, Kp], s_x float32 [M]."""
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(x_q, torch.int8, (M, bitnet_k_pad(K)), "x_q")
    _need(s_x, torch.float32, (M,), "s_x")
    _check(lib().bitnet_act_quant(_ptr(x), M, K, _ptr(x_q), _ptr(s_x), _stream(stream)))


def bitlinear_fwd(x_q, s_x, w_packed, gamma, K, y, acc_out=None, workspace=None, stream=None, bias=None):
    """INT8 forward: y [M, N] bf16 (and optionally acc_out int32 [M, N]);
    with `bias` (bf16 [N]) the bias is added before the rounding
    (bitlinear_fwd_bias)."""
    M, Kp = x_q.shape
    N = w_packed.shape[0]
    if Kp != bitnet_k_pad(K):
        raise ValueError("x_q: second dimension must be bitnet_k_pad(K)")
    _need(x_q, torch.int8, (M, Kp), "x_q")
    _need(s_x, torch.float32, (M,), "s_x")
    _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    _need(gamma, torch.float32, (1,), "gamma")
    _need(y, torch.bfloat16, (M, N), "y")
    if acc_out is not None:
        _need(acc_out, torch.int32, (M, N), "acc_out")
    if bias is not None:
        _need(bias, torch.bfloat16, (N,), "bias")
    if workspace is None:
        workspace = _workspace(bitlinear_fwd_workspace_bytes(M, N, K), y, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if bias is None:
        _check(lib().bitlinear_fwd(_ptr(x_q), _ptr(s_x), _ptr(w_packed), _ptr(gamma), M, N, int(K),
                                   _ptr(y), _ptr(acc_out), _ptr(workspace), ws_bytes, _stream(stream)))
    else:
        _check(lib().bitlinear_fwd_bias(_ptr(x_q), _ptr(s_x), _ptr(w_packed), _ptr(gamma), _ptr(bias), M, N,
                                        int(K), _ptr(y), _ptr(acc_out), _ptr(workspace), ws_bytes,
                                        _stream(stream)))


def bitlinear_bias_grad(dY, db, stream=None):
    """db [N] (float32 or bf16) = the token sum of dY [M, N] bf16."""
    M, N = dY.shape
    _need(dY, torch.bfloat16, (M, N), "dY")
    if db.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("db: expected float32 or bfloat16")
    _need(db, db.dtype, (N,), "db")
    dt = BITNET_F32 if db.dtype == torch.float32 else BITNET_BF16
    _check(lib().bitlinear_bias_grad(_ptr(dY), M, N, _ptr(db), dt, _stream(stream)))


def bitlinear_bwd(dY, x_q, s_x, w_packed, gamma, K, dX=None, dW=None, workspace=None, stream=None):
    """STE backward: dX [M, K] bf16 and/or dW [N, K] (bf16 or float32), or
    dW as 1-bit signs (uint8 [N, Kp/8]; bit j of byte b of row n set iff
    dW[n, 8b + j] < 0)."""
    M, N = dY.shape
    Kp = bitnet_k_pad(K)
    _need(dY, torch.bfloat16, (M, N), "dY")
    if dX is not None:
        _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
        _need(gamma, torch.float32, (1,), "gamma")
        _need(dX, torch.bfloat16, (M, int(K)), "dX")
    dw_dtype = BITNET_BF16
    if dW is not None:
        _need(x_q, torch.int8, (M, Kp), "x_q")
        _need(s_x, torch.float32, (M,), "s_x")
        if dW.dtype == torch.uint8:
            dw_dtype = BITNET_SIGN1
            _need(dW, torch.uint8, (N, Kp // 8), "dW")
        else:
            if dW.dtype == torch.float32:
                dw_dtype = BITNET_F32
            _need(dW, dW.dtype, (N, int(K)), "dW")
            if dW.dtype not in (torch.bfloat16, torch.float32):
                raise TypeError("dW: expected bfloat16, float32 or uint8 (1-bit signs)")
    if workspace is None:
        workspace = _workspace(bitlinear_bwd_workspace_bytes(M, N, K), dY, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bitlinear_bwd(_ptr(dY), _ptr(x_q), _ptr(s_x), _ptr(w_packed), _ptr(gamma),
                               M, N, int(K), _ptr(dX), _ptr(dW), dw_dtype, _ptr(workspace), ws_bytes,
                               _stream(stream)))


# --- TTQ ---------------------------------------------------------------------

def ttq_workspace_bytes(M, N, K):
    return int(lib().ttq_workspace_bytes(int(M), int(N), int(K)))


def _w_dtype(W):
    if W.dtype == torch.bfloat16:
        return BITNET_BF16
    if W.dtype == torch.float32:
        return BITNET_F32
    raise TypeError(f"W: expected bfloat16 or float32, got {W.dtype}")


def ttq_init(W, params, workspace, stream=None):
    """W [N, K] bf16 or float32 -> params float32 [3] = (delta, Wp, Wn)."""
    N, K = W.shape
    wd = _w_dtype(W)
    _need(W, W.dtype, (N, K), "W")
    _need(params, torch.float32, (3,), "params")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().ttq_init(_ptr(W), wd, N, K, _ptr(params), _ptr(workspace), ws_bytes, _stream(stream)))


def ttq_quantize(W, params, w_packed, wt, stream=None):
    """W [N, K], params (delta, Wp, Wn) -> codes uint8 [N, Kp/4] and bf16
    values wt [N, Kp]."""
    N, K = W.shape
    Kp = bitnet_k_pad(K)
    wd = _w_dtype(W)
    _need(W, W.dtype, (N, K), "W")
    _need(params, torch.float32, (3,), "params")
    _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    _need(wt, torch.bfloat16, (N, Kp), "wt")
    _check(lib().ttq_quantize(_ptr(W), wd, N, K, _ptr(params), _ptr(w_packed), _ptr(wt), _stream(stream)))


def ttq_fwd(x, wt, y, workspace=None, stream=None):
    """y [M, N] bf16 = x [M, K] bf16 @ wt[:, :K]^T."""
    M, K = x.shape
    N, Kp = wt.shape
    if Kp != bitnet_k_pad(K):
        raise ValueError("wt: second dimension must be bitnet_k_pad(K)")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(wt, torch.bfloat16, (N, Kp), "wt")
    _need(y, torch.bfloat16, (M, N), "y")
    if workspace is None:
        workspace = _workspace(ttq_workspace_bytes(M, N, K), y, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ttq_fwd(_ptr(x), _ptr(wt), M, N, K, _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))


def ttq_fwd_codes_workspace_bytes(M, N, K):
    return int(lib().ttq_fwd_codes_workspace_bytes(int(M), int(N), int(K)))


def ttq_fwd_codes(x, w_packed, params, y, workspace=None, stream=None):
    """y [M, N] bf16 from x [M, K] bf16, the codes uint8 [N, Kp/4] and params
    float32 [3] = (delta, Wp, Wn)."""
    M, K = x.shape
    N = w_packed.shape[0]
    Kp = bitnet_k_pad(K)
    _need(x, torch.bfloat16, (M, K), "x")
    _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    _need(params, torch.float32, (3,), "params")
    _need(y, torch.bfloat16, (M, N), "y")
    if workspace is None:
        workspace = _workspace(ttq_fwd_codes_workspace_bytes(M, N, K), y, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ttq_fwd_codes(_ptr(x), _ptr(w_packed), _ptr(params), M, N, K, _ptr(y), _ptr(workspace), ws_bytes,
                               _stream(stream)))


def ttq_bwd(dY, x, wt, w_packed, K, dX=None, dW=None, grads=None, workspace=None, stream=None):
    """dX [M, K] bf16, dW [N, K] (bf16 or float32) and grads float32 [2] =
    (dL/dWp, dL/dWn), each optional (grads needs dW)."""
    M, N = dY.shape
    Kp = bitnet_k_pad(K)
    _need(dY, torch.bfloat16, (M, N), "dY")
    if dX is not None:
        _need(wt, torch.bfloat16, (N, Kp), "wt")
        _need(dX, torch.bfloat16, (M, int(K)), "dX")
    dw_dtype = BITNET_BF16
    if dW is not None:
        _need(x, torch.bfloat16, (M, int(K)), "x")
        if dW.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("dW: expected bfloat16 or float32")
        _need(dW, dW.dtype, (N, int(K)), "dW")
        dw_dtype = BITNET_F32 if dW.dtype == torch.float32 else BITNET_BF16
    if grads is not None:
        _need(grads, torch.float32, (2,), "grads")
        _need(w_packed, torch.uint8, (N, Kp // 4), "w_packed")
    if workspace is None:
        workspace = _workspace(ttq_workspace_bytes(M, N, K), dY, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ttq_bwd(_ptr(dY), _ptr(x), _ptr(wt), _ptr(w_packed), M, N, int(K), _ptr(dX), _ptr(dW),
                         dw_dtype, _ptr(grads), _ptr(workspace), ws_bytes, _stream(stream)))


# --- test hooks --------------------------------------------------------------

def bitnet_set_test_knobs(split_ctas=0, pair_cols=0, no_skinny=0, spin_limit=None):
    """Process-wide launch knobs (see the header); no arguments restores the
    defaults (cost models, default spin limit)."""
    L = lib()
    if spin_limit is None:
        spin_limit = int(L.bitnet_default_spin_limit())
    L.bitnet_set_test_knobs(int(split_ctas), int(pair_cols), int(no_skinny), int(spin_limit))


def bitnet_split_timeouts():
    """Waits for partial tiles that gave up since the last call (synchronizes
    the device)."""
    c = ctypes.c_uint32(0)
    _check(lib().bitnet_split_timeouts(ctypes.byref(c)))
    return int(c.value)


def bitnet_quantize_recomputes():
    """Partial sums one-pass quantize launches computed themselves after
    their wait gave up, since the last call (synchronizes the device)."""
    c = ctypes.c_uint32(0)
    _check(lib().bitnet_quantize_recomputes(ctypes.byref(c)))
    return int(c.value)


def bitnet_debug_split_pieces(tiles, stages, grid):
    """The pieces of a split launch, as numpy arrays keyed v, t, s0, s1,
    slot, va, n (host-side computation; no GPU needed)."""
    import numpy as np

    L = lib()
    cap = int(grid) + int(tiles) + 1
    arrs = {k: np.zeros(cap, dtype=np.int32) for k in ("v", "t", "s0", "s1", "va", "n")}
    arrs["slot"] = np.zeros(cap, dtype=np.int64)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    n = int(L.bitnet_debug_split_pieces(int(tiles), int(stages), int(grid), ptr(arrs["v"]), ptr(arrs["t"]),
                                        ptr(arrs["s0"]), ptr(arrs["s1"]), ptr(arrs["slot"]), ptr(arrs["va"]),
                                        ptr(arrs["n"]), cap))
    if n < 0 or n > cap:
        raise ValueError(f"bitnet_debug_split_pieces({tiles}, {stages}, {grid}) returned {n}")
    return {k: a[:n] for k, a in arrs.items()}


def bitnet_debug_partial_slots(tiles, grid):
    return int(lib().bitnet_debug_partial_slots(int(tiles), int(grid)))


def bitnet_debug_cta_order(grid):
    import numpy as np

    out = np.zeros(int(grid), dtype=np.int32)
    lib().bitnet_debug_cta_order(int(grid), out.ctypes.data_as(ctypes.c_void_p))
    return out


def bitnet_debug_mfma_probe(int8, iters, sink, stream=None):
    """Enqueue the MFMA rate probe; returns the operations it performs.
    sink: float32 [2048] on the GPU."""
    _need(sink, torch.float32, (2048,), "sink")
    ops = ctypes.c_double(0.0)
    _check(lib().bitnet_debug_mfma_probe(1 if int8 else 0, int(iters), _ptr(sink), ctypes.byref(ops), _stream(stream)))
    return float(ops.value)
