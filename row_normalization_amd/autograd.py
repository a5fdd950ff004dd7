"""PyTorch autograd adapter over the C ABI (training use).

The adapter follows the shape the pages give for wiring the kernels into
autograd: the Triton RMSNorm tutorial (partitech.com), section "Kết nối
Autograd và thực sự huấn luyện" (a ``torch.autograd.Function`` whose forward
saves x, gamma and the inverse RMS for the backward, whose backward returns
one gradient per forward input, and a call counter that shows the kernel path
was taken), and the Unsloth walkthrough's ``fast_rms_layernorm`` wrapper
(section 3; the Gemma weight 1 + gamma).  The LayerNorm adapter has the
interface of the LayerNorm chapter (chuoer47.github.io), section 2: a
``torch.autograd.Function`` called as ``layernorm(x, normalized_shape, weight,
bias, eps)`` that saves x, weight, bias, mean and rstd and returns
(dx, None, dw, db, None).  The RoPE adapter follows the walkthrough's
section 4 (rotate q in place, save only the tables, rotate the gradient back
with the same kernel); the SwiGLU adapter its section 5 (the forward kernel,
and one backward kernel giving both input gradients).

Every computation runs in the HIP kernels (``rmsnorm_fwd``, ``rmsnorm_bwd``);
this module allocates outputs with torch and marshals arguments.  Inputs of
any leading shape are flattened to rows of the last dimension, which must be
contiguous.  The weight gradient is accumulated in fp32 by the library and
cast to gamma's dtype here, because autograd requires a gradient of the
parameter's own dtype (``rmsnorm_bwd`` gives the fp32 values directly).

The functional forms are excluded from ``torch.compile`` tracing
(``torch.compiler.disable``), as the walkthrough does for its kernels: the
calls go through ctypes into the library, which Dynamo cannot trace, so a
compiled model runs them eagerly between its compiled regions.
"""
from __future__ import annotations

import torch

from ._lib import (layernorm_bwd, layernorm_bwd_workspace_bytes, layernorm_fwd, rmsnorm_bwd,
                   rmsnorm_bwd_workspace_bytes, rmsnorm_fwd, rope_bwd, rope_fwd, swiglu_bwd, swiglu_fwd)

# Passes through the adapters (not kernel launches): forward and backward,
# RMSNorm and LayerNorm counted apart.
CALLS = {"forward": 0, "backward": 0, "ln_forward": 0, "ln_backward": 0, "rope_forward": 0, "rope_backward": 0,
         "swiglu_forward": 0, "swiglu_backward": 0}


def _rows(t: torch.Tensor) -> torch.Tensor:
    """[..., N] -> dense [M, N] rows (a copy only if t's rows are strided or spaced).

    The outputs the adapters allocate are dense, and the C ABI takes one row
    stride for all row operands, so the input rows must be dense too."""
    if t.dim() == 0:
        raise ValueError("RMSNorm needs at least one dimension")
    t2 = t.reshape(-1, t.shape[-1])
    if (t2.shape[1] > 1 and t2.stride(1) != 1) or (t2.shape[0] > 1 and t2.stride(0) != t2.shape[1]):
        t2 = t2.contiguous()
    return t2


class RMSNormFunction(torch.autograd.Function):
    """y = x * r * w with r = 1/sqrt(mean(x^2) + eps), w = gamma or 1 + gamma."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, gemma: bool = False,
                round_normed: bool = False):
        x2 = _rows(x)
        y = torch.empty(x2.shape, dtype=x.dtype, device=x.device)
        rstd = torch.empty(x2.shape[0], dtype=torch.float32, device=x.device)
        rmsnorm_fwd(x2, gamma, y, rstd, eps=eps, gemma=gemma, round_normed=round_normed)
        ctx.save_for_backward(x2, gamma, rstd)
        ctx.gemma = bool(gemma)
        ctx.x_shape = x.shape
        CALLS["forward"] += 1
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, gamma, rstd = ctx.saved_tensors
        M, N = x2.shape
        # the C ABI takes one row stride for x, dy and dx: dense rows (x2 was
        # made dense in the forward; dy.contiguous() as on the tutorial)
        dy2 = dy.reshape(M, N).contiguous()
        dx = torch.empty_like(dy2)
        dgamma = torch.empty(N, dtype=torch.float32, device=dy.device)
        ws_bytes = rmsnorm_bwd_workspace_bytes(M, N, x2.dtype)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dy.device)
        rmsnorm_bwd(x2, gamma, dy2, rstd, dx, dgamma, ws, gemma=ctx.gemma)
        CALLS["backward"] += 1
        return dx.view(ctx.x_shape), dgamma.to(gamma.dtype), None, None, None


@torch.compiler.disable
def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, gemma: bool = False,
            round_normed: bool = False) -> torch.Tensor:
    """Functional form: RMSNorm over the last dimension of x.

    ``round_normed`` rounds x * r to x's dtype before the weight multiply (the
    Hugging Face order); the gradient formula treats that rounding as the
    identity."""
    return RMSNormFunction.apply(x, gamma, eps, gemma, round_normed)


class RMSNorm(torch.nn.Module):
    """RMSNorm layer over the last dimension (weight initialised to 1, or 0 for Gemma's 1 + gamma)."""

    def __init__(self, hidden: int, eps: float = 1e-6, gemma: bool = False, round_normed: bool = False,
                 dtype=torch.bfloat16, device=None):
        super().__init__()
        init = torch.zeros if gemma else torch.ones
        self.weight = torch.nn.Parameter(init(hidden, dtype=dtype, device=device))
        self.eps = eps
        self.gemma = gemma
        self.round_normed = round_normed

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return rmsnorm(x, self.weight, self.eps, self.gemma, self.round_normed)

    def extra_repr(self) -> str:
        return f"{self.weight.shape[0]}, eps={self.eps}, gemma={self.gemma}"


class LayerNormFunction(torch.autograd.Function):
    """y = (x - mean) * rstd * weight + bias over the last dimension."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, normalized_shape, weight: torch.Tensor, bias: torch.Tensor, eps: float = 1e-5):
        N = x.shape[-1]
        if tuple(normalized_shape) != (N,):
            raise ValueError("normalized_shape must be (x.shape[-1],): LayerNorm over the last dimension only")
        x2 = _rows(x)
        y = torch.empty(x2.shape, dtype=x.dtype, device=x.device)
        mean = torch.empty(x2.shape[0], dtype=torch.float32, device=x.device)
        rstd = torch.empty(x2.shape[0], dtype=torch.float32, device=x.device)
        layernorm_fwd(x2, weight, bias, y, mean, rstd, eps=eps)
        ctx.save_for_backward(x2, weight, bias, mean, rstd)
        ctx.x_shape = x.shape
        CALLS["ln_forward"] += 1
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, weight, bias, mean, rstd = ctx.saved_tensors
        M, N = x2.shape
        dy2 = dy.reshape(M, N).contiguous()
        dx = torch.empty_like(dy2)
        dw = torch.empty(N, dtype=torch.float32, device=dy.device)
        db = torch.empty(N, dtype=torch.float32, device=dy.device)
        ws_bytes = layernorm_bwd_workspace_bytes(M, N, x2.dtype)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dy.device)
        layernorm_bwd(x2, weight, dy2, mean, rstd, dx, dw, db, ws)
        CALLS["ln_backward"] += 1
        return dx.view(ctx.x_shape), None, dw.to(weight.dtype), db.to(bias.dtype), None


@torch.compiler.disable
def layernorm(x: torch.Tensor, normalized_shape, weight: torch.Tensor, bias: torch.Tensor,
              eps: float = 1e-5) -> torch.Tensor:
    """Functional form with the signature of ``torch.nn.functional.layer_norm``
    (weight and bias required; normalisation over the last dimension)."""
    return LayerNormFunction.apply(x, normalized_shape, weight, bias, eps)


class LayerNorm(torch.nn.Module):
    """LayerNorm layer over the last dimension (weight initialised to 1, bias to 0)."""

    def __init__(self, hidden: int, eps: float = 1e-5, dtype=torch.float16, device=None):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.ones(hidden, dtype=dtype, device=device))
        self.bias = torch.nn.Parameter(torch.zeros(hidden, dtype=dtype, device=device))
        self.eps = eps

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return layernorm(x, (x.shape[-1],), self.weight, self.bias, self.eps)

    def extra_repr(self) -> str:
        return f"{self.weight.shape[0]}, eps={self.eps}"


class RoPEFunction(torch.autograd.Function):
    """Rotary embedding of q [tokens, heads, head_dim], in place (q is marked
    dirty and returned); the backward rotates the gradient back."""

    @staticmethod
    def forward(ctx, q: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, positions=None, seq_len=None):
        rope_fwd(q, cos, sin, positions, seq_len)
        ctx.mark_dirty(q)
        ctx.save_for_backward(cos, sin, positions)
        ctx.seq_len = seq_len
        CALLS["rope_forward"] += 1
        return q

    @staticmethod
    def backward(ctx, dq: torch.Tensor):
        cos, sin, positions = ctx.saved_tensors
        dq = dq.contiguous().clone()  # the incoming gradient may be shared: rotate a private copy in place
        rope_bwd(dq, cos, sin, positions, ctx.seq_len)
        CALLS["rope_backward"] += 1
        return dq, None, None, None, None


@torch.compiler.disable
def rope_embedding(q: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, positions=None, seq_len=None):
    """In-place rotary embedding of q [tokens, heads, head_dim] (see RoPEFunction)."""
    return RoPEFunction.apply(q, cos, sin, positions, seq_len)


class SwiGLUFunction(torch.autograd.Function):
    """h = T(T(silu(e)) * g) over [M, N]; the backward gives de and dg from one kernel."""

    @staticmethod
    def forward(ctx, e: torch.Tensor, g: torch.Tensor):
        shape = e.shape
        e2, g2 = e.reshape(-1, shape[-1]).contiguous(), g.reshape(-1, shape[-1]).contiguous()
        h = torch.empty_like(e2)
        swiglu_fwd(e2, g2, h)
        ctx.save_for_backward(e2, g2)
        ctx.shape = shape
        CALLS["swiglu_forward"] += 1
        return h.view(shape)

    @staticmethod
    def backward(ctx, dh: torch.Tensor):
        e2, g2 = ctx.saved_tensors
        dh2 = dh.reshape(e2.shape).contiguous()
        h = torch.empty_like(e2)
        dg = torch.empty_like(e2)
        de = torch.empty_like(e2)
        swiglu_bwd(dh2, e2, g2, h, dg, de)
        CALLS["swiglu_backward"] += 1
        return de.view(ctx.shape), dg.view(ctx.shape)


@torch.compiler.disable
def swiglu(e: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    """Elementwise SwiGLU h = silu(e) * g with autograd (see SwiGLUFunction)."""
    return SwiGLUFunction.apply(e, g)
