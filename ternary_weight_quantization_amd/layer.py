"""torch autograd wrapper and drop-in module over the C ABI.

``QATBitLinear`` mirrors the layer of the "bitnet-qat-train" page (Usage:
bf16 master weights [out, in], ``y = layer(x)``, STE gradients on
``layer.weight``; ``from_linear``; ``export_inference`` returning the packed
weights and their scale). The forward saves only the int8 activations, their
scales, the 2-bit weights and gamma ("bitnet-qat-train", opening bullets);
the backward rebuilds the operands from them inside the library's kernels.
``freeze`` / ``unfreeze`` and ``ternary_stats`` follow the BitLinear module of
"bitlinear.py": a frozen layer keeps its ternary weights and scale and runs
forward from them without re-ternarizing the masters. torch provides memory
and the stream; every step runs in libbitnet.so.
"""

import math

import torch

from . import binding as B


def ternarize(weight):
    """weight [N, K] (bf16 or f32, on the GPU) -> (w_packed uint8 [N, Kp/4],
    gamma float32 [1])."""
    N, K = weight.shape
    Kp = B.bitnet_k_pad(K)
    w_packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=weight.device)
    gamma = torch.empty((1,), dtype=torch.float32, device=weight.device)
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=weight.device)
    B.bitnet_ternarize_pack(weight.contiguous(), w_packed, gamma, ws)
    return w_packed, gamma


def act_quant(x2d):
    """x [M, K] bf16 -> (x_q int8 [M, Kp], s_x float32 [M])."""
    M, K = x2d.shape
    x_q = torch.empty((M, B.bitnet_k_pad(K)), dtype=torch.int8, device=x2d.device)
    s_x = torch.empty((M,), dtype=torch.float32, device=x2d.device)
    B.bitnet_act_quant(x2d, x_q, s_x)
    return x_q, s_x


def quantize(weight, x2d):
    """ternarize(weight) and act_quant(x2d) in one library call (the
    weight's absmean pass and the activation quantization share a launch):
    (w_packed, gamma, x_q, s_x)."""
    N, K = weight.shape
    M = x2d.shape[0]
    Kp = B.bitnet_k_pad(K)
    dev = weight.device
    w_packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=dev)
    gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    x_q = torch.empty((M, Kp), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=dev)
    B.bitnet_quantize(weight.contiguous(), x2d, w_packed, gamma, x_q, s_x, ws)
    return w_packed, gamma, x_q, s_x


def _workspace(nbytes, device):
    return None if nbytes == 0 else torch.empty((nbytes,), dtype=torch.uint8, device=device)


class BitLinearFunction(torch.autograd.Function):
    """y = BitLinear(x, W) (+ bias) with the STE backward. x [..., K] bf16,
    W [N, K] bf16 or float32, bias [N] bf16 or None; y [..., N] bf16.
    Gradients: dX bf16, dW in W's dtype, db bf16 (token sum of dY)."""

    @staticmethod
    def forward(ctx, x, weight, bias=None):
        if x.dtype != torch.bfloat16:
            raise TypeError("BitLinear expects bf16 activations")
        N, K = weight.shape
        lead = x.shape[:-1]
        x2 = x.reshape(-1, K).contiguous()
        M = x2.shape[0]
        w_packed, gamma, x_q, s_x = quantize(weight, x2)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        B.bitlinear_fwd(x_q, s_x, w_packed, gamma, K, y,
                        workspace=_workspace(B.bitlinear_fwd_workspace_bytes(M, N, K), x.device),
                        bias=None if bias is None else bias.to(torch.bfloat16).contiguous())
        ctx.save_for_backward(x_q, s_x, w_packed, gamma)
        ctx.shape = (M, N, K, lead, weight.dtype, None if bias is None else bias.dtype)
        return y.reshape(*lead, N)

    @staticmethod
    def backward(ctx, dy):
        x_q, s_x, w_packed, gamma = ctx.saved_tensors
        M, N, K, lead, wdtype, bdtype = ctx.shape
        dY = dy.reshape(M, N).to(torch.bfloat16).contiguous()
        need_x, need_w = ctx.needs_input_grad[:2]
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device) if need_x else None
        dW = torch.empty((N, K), dtype=wdtype, device=dy.device) if need_w else None
        if dX is not None or dW is not None:
            B.bitlinear_bwd(dY, x_q, s_x, w_packed, gamma, K, dX=dX, dW=dW,
                            workspace=_workspace(B.bitlinear_bwd_workspace_bytes(M, N, K), dy.device))
        db = None
        if bdtype is not None and ctx.needs_input_grad[2]:
            db = torch.empty((N,), dtype=torch.float32, device=dy.device)
            B.bitlinear_bias_grad(dY, db)
            db = db.to(bdtype)
        return (None if dX is None else dX.reshape(*lead, K)), dW, db


def bitlinear_inference(x, w_packed, gamma, in_features, bias=None):
    """The forward from a stored ternary state, e.g. the pair
    ``export_inference`` returns: y = BitLinear(x) with w_packed uint8
    [N, Kp/4] and gamma float32 [1] as bitnet_ternarize_pack writes them, x
    [..., in_features] bf16, optional bf16 bias [N]. Differentiable in x
    (the STE dX from the same state); the weights get no gradient."""
    return FrozenBitLinearFunction.apply(x, w_packed, gamma, in_features, bias)


class FrozenBitLinearFunction(torch.autograd.Function):
    """The layer's forward from a cached (w_packed, gamma): per-token int8
    activations and the INT8 GEMM, with no ternarization of master weights.
    Backward: dX = dY W_hat from the same cached state (the STE through the
    activation quantizer), and the bias gradient; none for the weights."""

    @staticmethod
    def forward(ctx, x, w_packed, gamma, in_features, bias=None):
        if x.dtype != torch.bfloat16:
            raise TypeError("BitLinear expects bf16 activations")
        K, N = int(in_features), w_packed.shape[0]
        lead = x.shape[:-1]
        x2 = x.reshape(-1, K).contiguous()
        M = x2.shape[0]
        x_q, s_x = act_quant(x2)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        B.bitlinear_fwd(x_q, s_x, w_packed, gamma, K, y,
                        workspace=_workspace(B.bitlinear_fwd_workspace_bytes(M, N, K), x.device),
                        bias=None if bias is None else bias.to(torch.bfloat16).contiguous())
        ctx.save_for_backward(w_packed, gamma)
        ctx.shape = (M, N, K, lead, None if bias is None else bias.dtype)
        return y.reshape(*lead, N)

    @staticmethod
    def backward(ctx, dy):
        w_packed, gamma = ctx.saved_tensors
        M, N, K, lead, bdtype = ctx.shape
        dY = dy.reshape(M, N).to(torch.bfloat16).contiguous()
        dX = None
        if ctx.needs_input_grad[0]:
            dX = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device)
            B.bitlinear_bwd(dY, None, None, w_packed, gamma, K, dX=dX,
                            workspace=_workspace(B.bitlinear_bwd_workspace_bytes(M, N, K), dy.device))
            dX = dX.reshape(*lead, K)
        db = None
        if bdtype is not None and ctx.needs_input_grad[4]:
            db = torch.empty((N,), dtype=torch.float32, device=dy.device)
            B.bitlinear_bias_grad(dY, db)
            db = db.to(bdtype)
        return dX, None, None, None, db


class QATBitLinear(torch.nn.Module):
    """Ternary-weight, int8-activation linear layer for quantization-aware
    training. Master weights [out_features, in_features] in bf16 (or f32),
    kaiming-uniform(a=sqrt(5)) init as in "bitlinear.py" BitLinear.__init__,
    and, with bias=True, a zero-initialised bf16 bias added before the
    output rounding (as that layer's optional bias; "bitnet-qat-train" has
    none, the default)."""

    def __init__(self, in_features, out_features, device="cuda", dtype=torch.bfloat16, bias=False):
        super().__init__()
        self.in_features = in_features
        self.out_features = out_features
        w = torch.empty((out_features, in_features), dtype=torch.float32)
        torch.nn.init.kaiming_uniform_(w, a=math.sqrt(5))
        self.weight = torch.nn.Parameter(w.to(device=device, dtype=dtype))
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, device=device, dtype=torch.bfloat16))
                     if bias else None)
        self.register_buffer("_frozen_packed", None)
        self.register_buffer("_frozen_gamma", None)
        self._inference_mode = False

    @classmethod
    def from_linear(cls, linear, dtype=torch.bfloat16):
        m = cls(linear.in_features, linear.out_features, device=linear.weight.device, dtype=dtype,
                bias=linear.bias is not None)
        with torch.no_grad():
            m.weight.copy_(linear.weight.to(dtype))
            if linear.bias is not None:
                m.bias.copy_(linear.bias.to(torch.bfloat16))
        return m

    def forward(self, x):
        if self.frozen:
            return FrozenBitLinearFunction.apply(x, self._frozen_packed, self._frozen_gamma, self.in_features,
                                                 self.bias)
        return BitLinearFunction.apply(x, self.weight, self.bias)

    @torch.no_grad()
    def freeze(self):
        """Ternarize the current master weights once and run every later
        forward from that (w_packed, gamma), as "bitlinear.py" BitLinear.freeze
        locks its layer to the ternary weights for inference. The forward
        stays the W1.58/A8 one (int8 activations, INT8 GEMM): a frozen layer
        gives bit for bit the outputs of the training forward at the moment
        of freezing. The masters get no gradient while frozen."""
        self._frozen_packed, self._frozen_gamma = ternarize(self.weight.detach())
        self._inference_mode = True
        return self

    def unfreeze(self):
        """Back to training: every forward ternarizes the masters again."""
        self._inference_mode = False
        return self

    @property
    def frozen(self):
        return self._inference_mode and self._frozen_packed is not None

    @torch.no_grad()
    def export_inference(self):
        """(w_packed uint8 [out, Kp/4], gamma float32 [1]): the frozen state
        when frozen, else that of the current master weights."""
        if self.frozen:
            return self._frozen_packed, self._frozen_gamma
        return ternarize(self.weight.detach())

    @property
    @torch.no_grad()
    def ternary_stats(self):
        """Shares of the codes -1, 0 and +1 in the ternary weight the forward
        uses ("bitlinear.py", BitLinear.ternary_stats), counted on the GPU."""
        w_packed = self.export_inference()[0]
        counts = torch.empty((2,), dtype=torch.int64, device=w_packed.device)
        B.bitnet_code_counts(w_packed, self.in_features, counts)
        neg, pos = (int(v) for v in counts.cpu())
        n = self.out_features * self.in_features
        return {"neg1": neg / n, "zero": (n - neg - pos) / n, "pos1": pos / n}

    def extra_repr(self):
        r = f"{self.in_features}, {self.out_features}, dtype={self.weight.dtype}, bias={self.bias is not None}"
        return r + (", frozen=True" if self.frozen else "")
