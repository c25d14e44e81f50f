"""fp64 CPU oracle for the two steps either side of the mixer: the short
convolution on its q/k/v inputs and the gated RMSNorm on its output.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline may import this module; the product library and its Python binding
never do.  It shares no code with the GPU path.

Source: the AMD ROCm blog "Pretraining hybrid LLMs with Primus", "Recipe"
(Table 4, the FLA fusion row, which lists fused SwiGLU, RMSNorm, gated norm and
short conv kernels, and the epsilon row, 1e-6).  The pages name the two steps
but do not define them; the readings taken here are the plain ones:

  short conv   a causal depthwise convolution of width W over the tokens of
               each sequence, one filter per channel, tokens before the
               sequence start counting as zero, then SiLU:
                 pre[t, c] = sum_j w[c, j] x[t - (W - 1) + j, c]
                 y[t, c]   = pre[t, c] * sigmoid(pre[t, c])
  gated norm   per row (one token and head, d values) an RMSNorm with a
               per-channel weight, gated by SiLU of a second input z:
                 y = o / sqrt(mean(o^2) + eps) * w * silu(z)

Layouts: x, dy of the convolution are [B, T, D] (or one packed row [1, T, D]
with cu_seqlens); w is [D, W].  o, z, dy of the norm are [..., d]; w is [d].
Everything is computed in fp64 from whatever dtype comes in.
"""
import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: widen bf16, keep fp32 / fp64 as they are
        import torch

        x = x.detach().cpu()
        x = (x.float() if x.dtype == torch.bfloat16 else x).numpy()
    return np.asarray(x, dtype=np.float64)


def _sigmoid(p):
    return 1.0 / (1.0 + np.exp(-p))


def _sequences(B, T, cu):
    """(batch row, first token, end token) of each sequence."""
    if cu is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(_f64(cu), dtype=np.int64)
    return [(0, int(cu[s]), int(cu[s + 1])) for s in range(len(cu) - 1)]


def _pre(xs, w):
    """pre-activation of one sequence xs [L, D]: left-pad W - 1 zero tokens,
    then tap j of every channel multiplies the token W - 1 - j places back."""
    W = w.shape[1]
    L = xs.shape[0]
    xp = np.concatenate([np.zeros((W - 1, xs.shape[1])), xs], axis=0)
    pre = np.zeros_like(xs)
    for j in range(W):
        pre += w[:, j] * xp[j:j + L]
    return pre, xp


def short_conv(x, w, cu=None):
    """y = silu(causal depthwise conv(x, w)) per sequence."""
    x, w = _f64(x), _f64(w)
    B, T, _ = x.shape
    y = np.zeros_like(x)
    for b, a, e in _sequences(B, T, cu):
        pre, _ = _pre(x[b, a:e], w)
        y[b, a:e] = pre * _sigmoid(pre)
    return y


def short_conv_bwd(x, w, dy, cu=None):
    """Gradients (dx, dw) of L = sum(dy * short_conv(x, w)).

    With g = dy * silu'(pre), silu'(p) = s (1 + p (1 - s)), s = sigmoid(p):
      dx[t] = sum_j w[:, j] g[t + (W - 1) - j]   (g past the sequence end = 0)
      dw[:, j] = sum over every sequence and token t of g[t] x[t - (W - 1) + j]
    """
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    B, T, D = x.shape
    W = w.shape[1]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for b, a, e in _sequences(B, T, cu):
        L = e - a
        pre, xp = _pre(x[b, a:e], w)
        s = _sigmoid(pre)
        g = dy[b, a:e] * (s * (1.0 + pre * (1.0 - s)))
        gp = np.concatenate([g, np.zeros((W - 1, D))], axis=0)
        for j in range(W):
            dx[b, a:e] += w[:, j] * gp[W - 1 - j:W - 1 - j + L]
            dw[:, j] += np.sum(g * xp[j:j + L], axis=0)
    return dx, dw


def gated_rmsnorm(o, z, w, eps=1e-6):
    """y = o / sqrt(mean(o^2) + eps) * w * silu(z), over the last axis."""
    o, z, w = _f64(o), _f64(z), _f64(w)
    rstd = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * rstd * w * (z * _sigmoid(z))


def gated_rmsnorm_bwd(o, z, w, dy, eps=1e-6):
    """Gradients (do, dz, dw) of L = sum(dy * gated_rmsnorm(o, z, w)).

    With r = 1 / sqrt(mean(o^2) + eps), n = o r, s = sigmoid(z):
      dz = dy n w s (1 + z (1 - s))
      dn = dy w z s,  do = r (dn - n mean(dn n))
      dw = sum over rows of dy n z s
    """
    o, z, w, dy = _f64(o), _f64(z), _f64(w), _f64(dy)
    d = o.shape[-1]
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    n = o * r
    s = _sigmoid(z)
    dz = dy * n * w * (s * (1.0 + z * (1.0 - s)))
    dn = dy * w * z * s
    do = r * (dn - n * np.sum(dn * n, axis=-1, keepdims=True) / d)
    dw = np.sum((dy * n * z * s).reshape(-1, d), axis=0)
    return do, dz, dw
