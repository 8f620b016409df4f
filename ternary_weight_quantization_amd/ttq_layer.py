"""torch autograd wrapper and module for the TTQ variant over the C ABI.

Trained ternary quantization as the "TTQ_VERIFICATION.md" page describes it
(LabStrangeLoop bitnet, after Zhu et al.): the weight is +Wp where the latent
weight exceeds a threshold delta, -Wn below -delta and 0 elsewhere (Eq. 1);
delta, Wp and Wn are learned per layer, kept positive through softplus
("Key Design Decisions" item 1) and initialized so that after the transform
they equal 0.7 E|W|, E|W| and E|W| (Eq. 2; "Bugs Fixed" item 5: the raw
values are the inverse softplus of those). Activations are not quantized
("Bugs Fixed" item 4). The latent weight gets the quantized weight's
gradient unchanged (straight-through), Wp and Wn the masked sums of it.

torch provides memory, the stream and the three-scalar softplus of the
parametrization; the quantizer and the products run in libbitnet.so.
"""

import math

import torch

from . import binding as B


def _inverse_softplus(v):
    # softplus(r) = log(1 + e^r) = v  <=>  r = v + log(1 - e^-v)
    return v + torch.log(-torch.expm1(-v))


def ttq_init(weight):
    """Initial (delta, Wp, Wn) float32 [3] of a latent weight [N, K] (Eq. 2),
    computed by the library."""
    N, K = weight.shape
    params = torch.empty((3,), dtype=torch.float32, device=weight.device)
    ws = torch.empty((B.bitnet_ternarize_workspace_bytes(N, K),), dtype=torch.uint8, device=weight.device)
    B.ttq_init(weight.contiguous(), params, ws)
    return params


def ttq_quantize(weight, params):
    """(w_packed uint8 [N, Kp/4], wt bf16 [N, Kp]) of Eq. 1 for params
    (delta, Wp, Wn) float32 [3] on the device."""
    N, K = weight.shape
    Kp = B.bitnet_k_pad(K)
    w_packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=weight.device)
    wt = torch.empty((N, Kp), dtype=torch.bfloat16, device=weight.device)
    B.ttq_quantize(weight.contiguous(), params.contiguous(), w_packed, wt)
    return w_packed, wt


def ttq_forward_codes(x, w_packed, params):
    """Inference forward from the exported state (``TTQLinear.export_inference``):
    x [..., K] bf16, codes [N, Kp/4], params (delta, Wp, Wn) -> y [..., N]
    bf16. Few tokens read only the 2-bit codes."""
    K = x.shape[-1]
    lead = x.shape[:-1]
    x2 = x.reshape(-1, K).contiguous()
    y = torch.empty((x2.shape[0], w_packed.shape[0]), dtype=torch.bfloat16, device=x.device)
    B.ttq_fwd_codes(x2, w_packed, params.contiguous(), y)
    return y.reshape(*lead, w_packed.shape[0])


def _workspace(nbytes, device):
    return None if nbytes == 0 else torch.empty((nbytes,), dtype=torch.uint8, device=device)


class TTQFunction(torch.autograd.Function):
    """y = x @ W_t^T with W_t from Eq. 1. x [..., K] bf16, weight [N, K] bf16
    or float32, params float32 [3] = (delta, Wp, Wn), already positive.
    Gradients: dX bf16, dW in the weight's dtype, d params =
    (0, dL/dWp, dL/dWn) (the threshold gets none)."""

    @staticmethod
    def forward(ctx, x, weight, params):
        if x.dtype != torch.bfloat16:
            raise TypeError("TTQ expects bf16 activations")
        N, K = weight.shape
        lead = x.shape[:-1]
        x2 = x.reshape(-1, K).contiguous()
        M = x2.shape[0]
        params = params.detach().to(torch.float32).contiguous()
        w_packed, wt = ttq_quantize(weight.detach(), params)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        ws = _workspace(B.ttq_workspace_bytes(M, N, K), x.device)
        B.ttq_fwd(x2, wt, y, workspace=ws)
        ctx.save_for_backward(x2, wt, w_packed)
        ctx.shape = (M, N, K, lead, weight.dtype)
        return y.reshape(*lead, N)

    @staticmethod
    def backward(ctx, dy):
        x2, wt, w_packed = ctx.saved_tensors
        M, N, K, lead, wdtype = ctx.shape
        dY = dy.reshape(M, N).to(torch.bfloat16).contiguous()
        need_x, need_w, need_p = ctx.needs_input_grad[:3]
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device) if need_x else None
        # the scale gradients come from dW's epilogue, so dW is computed
        # whenever either is needed
        dW = torch.empty((N, K), dtype=wdtype, device=dy.device) if (need_w or need_p) else None
        dparams = torch.zeros((3,), dtype=torch.float32, device=dy.device) if need_p else None
        if dX is not None or dW is not None:
            B.ttq_bwd(dY, x2, wt, w_packed, K, dX=dX, dW=dW, grads=None if dparams is None else dparams[1:],
                      workspace=_workspace(B.ttq_workspace_bytes(M, N, K), dy.device))
        return (None if dX is None else dX.reshape(*lead, K)), (dW if need_w else None), dparams


class TTQLinear(torch.nn.Module):
    """Linear layer with TTQ weights: latent weights [out, in] (bf16 or f32,
    kaiming-uniform(a=sqrt(5)) init like QATBitLinear) and three raw scalars
    whose softplus gives delta, Wp and Wn, initialized from the weights by
    the library (Eq. 2)."""

    def __init__(self, in_features, out_features, device="cuda", dtype=torch.bfloat16):
        super().__init__()
        self.in_features = in_features
        self.out_features = out_features
        w = torch.empty((out_features, in_features), dtype=torch.float32)
        torch.nn.init.kaiming_uniform_(w, a=math.sqrt(5))
        self.weight = torch.nn.Parameter(w.to(device=device, dtype=dtype))
        self.raw = torch.nn.Parameter(torch.zeros(3, dtype=torch.float32, device=device))
        self.reset_scales()

    @torch.no_grad()
    def reset_scales(self):
        """raw = inverse softplus of the Eq. 2 values of the current weight."""
        self.raw.copy_(_inverse_softplus(ttq_init(self.weight.detach()).double()).float())

    @classmethod
    def from_linear(cls, linear, dtype=torch.bfloat16):
        m = cls(linear.in_features, linear.out_features, device=linear.weight.device, dtype=dtype)
        with torch.no_grad():
            m.weight.copy_(linear.weight.to(dtype))
        m.reset_scales()
        return m

    def params(self):
        """(delta, Wp, Wn) float32 [3], positive."""
        return torch.nn.functional.softplus(self.raw)

    def forward(self, x):
        return TTQFunction.apply(x, self.weight, self.params())

    @torch.no_grad()
    def export_inference(self):
        """(w_packed uint8 [out, Kp/4], params float32 [3] = (delta, Wp, Wn)):
        the codes and the values they stand for."""
        p = self.params().detach().contiguous()
        return ttq_quantize(self.weight.detach(), p)[0], p

    def extra_repr(self):
        return f"{self.in_features}, {self.out_features}, dtype={self.weight.dtype}"
