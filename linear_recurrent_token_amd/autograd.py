"""torch.autograd bindings of liblrt.so: each forward is the library's training
forward, which leaves in its workspace what the backward would recompute, and
each backward is the matching ``*_bwd_saved`` entry point on that workspace.
Marshalling only -- every step runs in the library's kernels (no CPU path).

    o, ht = gated_delta_net(q, k, v, log_a, beta, h0=None, chunk=64)
    o, ht = kimi_delta_attention(q, k, v, log_a, beta, h0=None, chunk=64)   # log_a [B, T, H, d_k]
    o, ht = mamba2(q, k, v, log_a, h0=None, chunk=64)
    y = short_conv(x, w, cu_seqlens=None)          # silu(causal depthwise conv), w fp32 [D, W]
    y = gated_rms_norm(o, z, w, eps=1e-6)          # o / rms(o) * w * silu(z), w fp32 [d]

Shapes, dtypes and conventions are those of include/lrt.h (q, k, v [B, T, H, d]
fp32 or bf16; gates, beta and states fp32).  Gradients flow to every tensor
input (h0 too when given); the chunk size and eps are not differentiable.
"""
import torch

from . import (gated_rmsnorm as _gnorm_fwd, gated_rmsnorm_bwd as _gnorm_bwd, gdn_bwd_saved, gdn_fwd_train,
               kda_bwd_saved, kda_fwd_train, short_conv as _conv_fwd, short_conv_bwd as _conv_bwd, ssd_bwd_saved,
               ssd_fwd_train)


def _grad(t, like):
    """An incoming gradient as the contiguous tensor of like's dtype the library takes."""
    return t.to(like.dtype).contiguous()


class _DeltaRule(torch.autograd.Function):
    """Gated DeltaNet (kda=False) or Kimi Delta Attention (kda=True)."""

    @staticmethod
    def forward(ctx, q, k, v, log_a, beta, h0, chunk, kda):
        fwd = kda_fwd_train if kda else gdn_fwd_train
        o, ht, saved = fwd(q, k, v, log_a, beta, h0, chunk=chunk)
        ctx.save_for_backward(q, k, v, log_a, beta, h0)
        ctx.saved_ws, ctx.chunk, ctx.kda, ctx.has_h0 = saved, chunk, kda, h0 is not None
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, log_a, beta, h0 = ctx.saved_tensors
        bwd = kda_bwd_saved if ctx.kda else gdn_bwd_saved
        dq, dk, dv, dla, db, dh0 = bwd(q, k, v, log_a, beta, h0, _grad(do, q), ctx.saved_ws,
                                       _grad(dht, log_a), chunk=ctx.chunk, want_dh0=ctx.has_h0)
        ctx.saved_ws = None
        return dq, dk, dv, dla, db, dh0, None, None


class _Mamba2(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, log_a, h0, chunk):
        o, ht, saved = ssd_fwd_train(q, k, v, log_a, h0, chunk=chunk)
        ctx.save_for_backward(q, k, v, log_a, h0)
        ctx.saved_ws, ctx.chunk, ctx.has_h0 = saved, chunk, h0 is not None
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, log_a, h0 = ctx.saved_tensors
        dq, dk, dv, dla, dh0 = ssd_bwd_saved(q, k, v, log_a, h0, _grad(do, q), ctx.saved_ws, _grad(dht, log_a),
                                             chunk=ctx.chunk, want_dh0=ctx.has_h0)
        ctx.saved_ws = None
        return dq, dk, dv, dla, dh0, None


class _ShortConv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, cu_seqlens):
        ctx.save_for_backward(x, w, cu_seqlens)
        return _conv_fwd(x, w, cu_seqlens=cu_seqlens)

    @staticmethod
    def backward(ctx, dy):
        x, w, cu = ctx.saved_tensors
        dx, dw = _conv_bwd(x, w, _grad(dy, x), cu_seqlens=cu)
        return dx, dw, None


class _GatedRMSNorm(torch.autograd.Function):
    @staticmethod
    def forward(ctx, o, z, w, eps):
        ctx.save_for_backward(o, z, w)
        ctx.eps = eps
        return _gnorm_fwd(o, z, w, eps=eps)

    @staticmethod
    def backward(ctx, dy):
        o, z, w = ctx.saved_tensors
        do, dz, dw = _gnorm_bwd(o, z, w, _grad(dy, o), eps=ctx.eps)
        return do, dz, dw, None


def gated_delta_net(q, k, v, log_a, beta, h0=None, chunk=64):
    """Gated DeltaNet with autograd -> (o, ht)."""
    return _DeltaRule.apply(q, k, v, log_a, beta, h0, chunk, False)


def kimi_delta_attention(q, k, v, log_a, beta, h0=None, chunk=64):
    """Kimi Delta Attention (per-dimension log_a [B, T, H, d_k]) with autograd -> (o, ht)."""
    return _DeltaRule.apply(q, k, v, log_a, beta, h0, chunk, True)


def mamba2(q, k, v, log_a, h0=None, chunk=64):
    """The Mamba2 (SSD) recurrence with autograd -> (o, ht)."""
    return _Mamba2.apply(q, k, v, log_a, h0, chunk)


def short_conv(x, w, cu_seqlens=None):
    """silu(causal depthwise conv(x, w)) with autograd; x [B, T, D], w fp32 [D, W]."""
    return _ShortConv.apply(x, w, cu_seqlens)


def gated_rms_norm(o, z, w, eps=1e-6):
    """o / sqrt(mean(o^2) + eps) * w * silu(z) with autograd; w fp32 [d]."""
    return _GatedRMSNorm.apply(o, z, w, eps)
