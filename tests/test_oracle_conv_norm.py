"""Pins of the fp64 oracle of the short convolution and the gated RMSNorm
(oracle/conv_norm.py) against what fixes them independently of its code:

  * the convolution per channel equals scipy.signal.lfilter's FIR filter with
    the taps reversed (zero initial conditions = zero tokens before the
    sequence), SiLU equals x * scipy.special.expit(x);
  * packed sequences restart the filter: each sequence alone gives the same;
  * the norm equals torch.nn.functional.rms_norm (fp64) times F.silu(z), and
    a constant row c has the closed form c / sqrt(c^2 + eps);
  * both backwards equal torch.autograd of the same ops built from torch's own
    conv1d / rms_norm (fp64, CPU) and central finite differences of the
    oracle's forward.
"""
import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch
import torch.nn.functional as F

from oracle import conv_norm as cn


def rng(seed):
    return np.random.default_rng(seed)


def test_short_conv_is_fir_filter_then_silu():
    r = rng(0)
    B, T, D, W = 2, 37, 6, 4
    x = r.standard_normal((B, T, D))
    w = r.standard_normal((D, W))
    y = cn.short_conv(x, w)
    for b in range(B):
        for c in range(D):
            pre = scipy.signal.lfilter(w[c, ::-1], [1.0], x[b, :, c])
            np.testing.assert_allclose(y[b, :, c], pre * scipy.special.expit(pre), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_short_conv_delta_filters_shift(W):
    """A filter with one tap at lag m (tap W - 1 - m) shifts the sequence by m."""
    r = rng(1)
    T, D = 11, 3
    x = r.standard_normal((1, T, D))
    for m in range(W):
        w = np.zeros((D, W))
        w[:, W - 1 - m] = 1.0
        pre = np.zeros_like(x)
        pre[:, m:] = x[:, :T - m]
        np.testing.assert_allclose(cn.short_conv(x, w), pre * scipy.special.expit(pre), rtol=0, atol=1e-15)


def test_short_conv_packed_restarts_per_sequence():
    r = rng(2)
    lens = [5, 1, 0, 9, 2]
    T, D, W = sum(lens), 4, 4
    x = r.standard_normal((1, T, D))
    w = r.standard_normal((D, W))
    cu = np.concatenate([[0], np.cumsum(lens)])
    y = cn.short_conv(x, w, cu=cu)
    dy = r.standard_normal((1, T, D))
    dx, dw = cn.short_conv_bwd(x, w, dy, cu=cu)
    dw_sum = np.zeros_like(w)
    for a, e in zip(cu[:-1], cu[1:]):
        if e == a:
            continue
        np.testing.assert_allclose(y[:, a:e], cn.short_conv(x[:, a:e], w), rtol=0, atol=0)
        dxs, dws = cn.short_conv_bwd(x[:, a:e], w, dy[:, a:e])
        np.testing.assert_allclose(dx[:, a:e], dxs, rtol=0, atol=0)
        dw_sum += dws
    np.testing.assert_allclose(dw, dw_sum, rtol=1e-13, atol=1e-13)


def torch_conv(x, w):
    """silu(conv1d) through torch's own depthwise conv1d (channels first)."""
    D, W = w.shape
    pre = F.conv1d(x.transpose(1, 2), w.view(D, 1, W), padding=W - 1, groups=D)[..., :x.shape[1]]
    return F.silu(pre).transpose(1, 2)


def test_short_conv_matches_torch_and_its_backward():
    r = rng(3)
    B, T, D, W = 2, 23, 5, 4
    x = torch.tensor(r.standard_normal((B, T, D)), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(r.standard_normal((D, W)), dtype=torch.float64, requires_grad=True)
    dy = torch.tensor(r.standard_normal((B, T, D)), dtype=torch.float64)
    y = torch_conv(x, w)
    np.testing.assert_allclose(cn.short_conv(x.detach(), w.detach()), y.detach().numpy(), rtol=1e-12, atol=1e-12)
    gx, gw = torch.autograd.grad(y, (x, w), dy)
    dx, dw = cn.short_conv_bwd(x.detach(), w.detach(), dy)
    np.testing.assert_allclose(dx, gx.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw, gw.numpy(), rtol=1e-11, atol=1e-11)


def test_short_conv_backward_finite_differences():
    r = rng(4)
    B, T, D, W = 1, 9, 3, 4
    x = r.standard_normal((B, T, D))
    w = r.standard_normal((D, W))
    dy = r.standard_normal((B, T, D))
    dx, dw = cn.short_conv_bwd(x, w, dy)
    h = 1e-6
    loss = lambda xx, ww: float(np.sum(dy * cn.short_conv(xx, ww)))
    for idx in [(0, 0, 0), (0, 4, 1), (0, 8, 2), (0, 6, 0)]:
        e = np.zeros_like(x)
        e[idx] = h
        num = (loss(x + e, w) - loss(x - e, w)) / (2 * h)
        assert abs(num - dx[idx]) < 1e-7 * max(1.0, abs(num))
    for idx in [(0, 0), (1, 3), (2, 1)]:
        e = np.zeros_like(w)
        e[idx] = h
        num = (loss(x, w + e) - loss(x, w - e)) / (2 * h)
        assert abs(num - dw[idx]) < 1e-7 * max(1.0, abs(num))


def test_gated_rmsnorm_matches_torch_and_closed_forms():
    r = rng(5)
    o = r.standard_normal((3, 4, 2, 16))
    z = r.standard_normal((3, 4, 2, 16))
    w = r.standard_normal(16)
    to = torch.tensor(o)
    ref = F.rms_norm(to, (16,), weight=torch.tensor(w), eps=1e-6) * F.silu(torch.tensor(z))
    np.testing.assert_allclose(cn.gated_rmsnorm(o, z, w), ref.numpy(), rtol=1e-12, atol=1e-12)
    # a constant row c: every normalised entry is c / sqrt(c^2 + eps)
    c, eps = 0.003, 1e-6
    y = cn.gated_rmsnorm(np.full((1, 8), c), np.full((1, 8), 50.0), np.ones(8), eps=eps)
    np.testing.assert_allclose(y, c / np.sqrt(c * c + eps) * 50.0 * scipy.special.expit(50.0), rtol=1e-13)
    # a zero gate closes the output
    assert np.all(cn.gated_rmsnorm(o, np.zeros_like(z), w) == 0.0)


def test_gated_rmsnorm_backward_matches_autograd_and_finite_differences():
    r = rng(6)
    o = torch.tensor(r.standard_normal((5, 3, 32)), requires_grad=True)
    z = torch.tensor(r.standard_normal((5, 3, 32)), requires_grad=True)
    w = torch.tensor(r.standard_normal(32), requires_grad=True)
    dy = torch.tensor(r.standard_normal((5, 3, 32)))
    y = F.rms_norm(o, (32,), weight=w, eps=1e-6) * F.silu(z)
    go, gz, gw = torch.autograd.grad(y, (o, z, w), dy)
    do, dz, dw = cn.gated_rmsnorm_bwd(o.detach(), z.detach(), w.detach(), dy)
    np.testing.assert_allclose(do, go.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dz, gz.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dw, gw.numpy(), rtol=1e-10, atol=1e-11)
    on, zn, wn, dyn = (t.detach().numpy() for t in (o, z, w, dy))
    loss = lambda a, b, c: float(np.sum(dyn * cn.gated_rmsnorm(a, b, c)))
    h = 1e-6
    for idx in [(0, 0, 0), (4, 2, 31), (2, 1, 7)]:
        e = np.zeros_like(on)
        e[idx] = h
        num = (loss(on + e, zn, wn) - loss(on - e, zn, wn)) / (2 * h)
        assert abs(num - do[idx]) < 1e-7 * max(1.0, abs(num))
        num = (loss(on, zn + e, wn) - loss(on, zn - e, wn)) / (2 * h)
        assert abs(num - dz[idx]) < 1e-7 * max(1.0, abs(num))
