"""`sdpa_bob`: softmax attention as a twice-differentiable PyTorch op over the
C ABI (fa_fwd, fa_bwd, fa_bob).

Source: [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward for
Softmax Attention", section 4.1: the backward-over-backward is the
vector-Jacobian product of the first backward (dQ, dK, dV) = f(Q, K, V, dO)
with cotangents (U_Q, U_K, U_V); sections 4.2-4.3 and appendix D give the
closed forms fa_bob evaluates.  Differentiating a loss through attention
twice -- a Hessian-vector product, or the gradient of any function of the
first gradients -- reaches exactly that product.

Two autograd nodes:

* ``_Attn``: forward = fa_fwd (O fp32, L saved); backward = ``_AttnBwd``, so
  that the first backward is itself differentiable;
* ``_AttnBwd``: forward = fa_bwd (dQ, dK, dV fp32); backward = fa_bob with
  (U_Q, U_K, U_V) = the incoming gradients of (dQ, dK, dV), returning the
  total derivatives with respect to Q, K, V and dO.  O and L are functions
  of (Q, K, V) whose dependence fa_bob already includes, so no gradient is
  returned for them.

Every step runs in the HIP kernels; this module only marshals tensors.  The
library takes dO and the cotangents in the input dtype, so for bf16 inputs
they are rounded to bf16 on the way in (as any bf16 attention kernel does);
outputs are fp32 and autograd casts input gradients to the inputs' dtype.
K and V may have fewer heads than Q (grouped-query / multi-query attention).
With a dropout rate, every call passes the same (rate, seed), so the forward,
the first backward and the BoB see one mask (the pages' analytical dropout
extension, appendix G).
"""
from __future__ import annotations

import torch

from . import fa_bob, fa_bwd, fa_fwd


class _NoThirdOrder(torch.autograd.Function):
    """Identity on x that makes x depend on `deps` and refuses to be
    differentiated: a third derivative through sdpa_bob is not provided, and
    without this node autograd would treat fa_bob's outputs as constants and
    return a wrong third derivative instead of an error."""

    @staticmethod
    def forward(ctx, x, *deps):
        return x.view_as(x)

    @staticmethod
    def backward(ctx, *grads):
        raise RuntimeError("sdpa_bob: derivatives beyond the second (backward-over-backward) are not provided")


class _Attn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, causal, dropout, seed):
        o, lse = fa_fwd(q, k, v, scale=scale, causal=causal, dropout=dropout, seed=seed)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal, ctx.drop = scale, causal, (dropout, seed)
        ctx.mark_non_differentiable(lse)
        # An absent gradient stays None (no zero-filled dO): _AttnBwd returns
        # none for O, and the first backward must not run again for nothing.
        ctx.set_materialize_grads(False)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        if do is None:
            return (None,) * 7
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = _AttnBwd.apply(q, k, v, o, lse, do.to(q.dtype), ctx.scale, ctx.causal, *ctx.drop)
        return dq, dk, dv, None, None, None, None


class _AttnBwd(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, o, lse, do, scale, causal, dropout, seed):
        dq, dk, dv, _ = fa_bwd(q, k, v, o, lse, do.contiguous(), scale=scale, causal=causal, dropout=dropout,
                               seed=seed)
        ctx.save_for_backward(q, k, v, o, lse, do)
        ctx.scale, ctx.causal, ctx.drop = scale, causal, (dropout, seed)
        ctx.set_materialize_grads(False)
        return dq, dk, dv

    @staticmethod
    def backward(ctx, uq, uk, uv):
        if uq is None and uk is None and uv is None:
            return (None,) * 10
        q, k, v, o, lse, do = ctx.saved_tensors
        dt = q.dtype

        def cot(u, like):
            return torch.zeros_like(like) if u is None else u.detach().to(dt).contiguous()

        with torch.no_grad():
            out = fa_bob(q, k, v, o, lse, do.contiguous(), cot(uq, q), cot(uk, k), cot(uv, v),
                         scale=ctx.scale, causal=ctx.causal, dropout=ctx.drop[0], seed=ctx.drop[1])[:4]
        deps = [t for t in (q, k, v, do, uq, uk, uv) if t is not None and t.requires_grad]
        if torch.is_grad_enabled() and deps:
            # The caller asked for a graph of these gradients (create_graph):
            # make any further differentiation fail loudly.
            out = [_NoThirdOrder.apply(x, *deps) for x in out]
        gq, gk, gv, gdo = out
        return gq, gk, gv, None, None, gdo, None, None, None, None


def sdpa_bob(q, k, v, scale=None, causal=False, dropout_p=0.0, seed=0):
    """O = softmax(scale q k^T [+ causal mask]) v for [B, H, N, d] tensors
    (bf16 or fp32; k, v with H or a divisor of H heads), differentiable twice
    through the library's kernels.  Returns O in fp32.  ``scale`` defaults to
    1/sqrt(d).  ``dropout_p`` > 0 applies the library's dropout mask for
    ``seed`` (O = (P * g) V); the same mask is used by both derivatives.  The
    rate is used as the nearest multiple of 1/256 (t = round(256 p) of 256
    generator bytes drop an element, so p = 0.1 drops 26/256 = 10.16 %), and a
    rate below 1/512 rounds to no dropout at all (the binding warns)."""
    for t in (q, k, v):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("q, k, v must be [B, H, N, d] with a contiguous head dimension")
    o, _ = _Attn.apply(q, k, v, scale, bool(causal), float(dropout_p), int(seed))
    return o
