"""GPU parity of the steps either side of the mixer -- short_conv_fwd/bwd and
gated_rmsnorm_fwd/bwd -- against the fp64 oracle (oracle/conv_norm.py),
through the C ABI.

Bar: max|got - oracle| / max|oracle| per output tensor <= 1e-4 for fp32
inputs and <= 1e-2 for bf16 inputs (the oracle is fed the same rounded
inputs; bf16 outputs are rounded once).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import conv_norm as cn

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def lrt():
    import linear_recurrent_token_amd as L
    L.lib()
    return L


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0)) if ref.size else 0.0


def gen(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


CONV = [
    # name, B, T, D, W, dtype
    ("fp32_T37_D64_W4", 2, 37, 64, 4, torch.float32),
    ("fp32_T5_D40_W3", 3, 5, 40, 3, torch.float32),  # fewer pieces than a wave's lanes, T < one block
    ("bf16_T300_D1024_W4", 1, 300, 1024, 4, torch.bfloat16),
    ("bf16_T16_D8_W2", 2, 16, 8, 2, torch.bfloat16),
    ("bf16_T129_D264_W3", 2, 129, 264, 3, torch.bfloat16),  # a partial piece group
    ("fp32_T1_D16_W4", 4, 1, 16, 4, torch.float32),
]


def conv_inputs(B, T, D, W, dt, seed):
    x = torch.randn((B, T, D), generator=gen(seed), device="cuda").to(dt)
    w = 0.5 * torch.randn((D, W), generator=gen(seed + 1), device="cuda")
    dy = torch.randn((B, T, D), generator=gen(seed + 2), device="cuda").to(dt)
    return x, w, dy


def check_conv(x, w, dy, dt, cu=None, label=""):
    L = lrt()
    y = L.short_conv(x, w, cu_seqlens=cu)
    dx, dw = L.short_conv_bwd(x, w, dy, cu_seqlens=cu)
    torch.cuda.synchronize()
    cun = None if cu is None else cu.cpu().numpy()
    ry = cn.short_conv(x, w, cu=cun)
    rdx, rdw = cn.short_conv_bwd(x, w, dy, cu=cun)
    errs = {"y": rel(f64(y), ry), "dx": rel(f64(dx), rdx), "dw": rel(f64(dw), rdw)}
    say(f"  {label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if v > TOL[dt]}
    assert not bad, bad
    return y, dx, dw


@pytest.mark.parametrize("case", CONV, ids=[c[0] for c in CONV])
def test_short_conv(case):
    name, B, T, D, W, dt = case
    say(f"[conv] {name}")
    x, w, dy = conv_inputs(B, T, D, W, dt, 10)
    check_conv(x, w, dy, dt, label=name)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_short_conv_packed(dt):
    """Packed sequences restart the filter at every boundary, including
    boundaries inside a 16-token block, one-token and empty sequences."""
    lens = [5, 1, 0, 9, 2, 40, 17, 33, 16]
    T, D, W = sum(lens), 72, 4
    say(f"[conv packed] {dt} lens={lens}")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    x, w, dy = conv_inputs(1, T, D, W, dt, 20)
    y, dx, dw = check_conv(x, w, dy, dt, cu=cu, label="packed")
    # each sequence alone through the dense call gives the same rows
    L = lrt()
    starts = np.concatenate([[0], np.cumsum(lens)])
    for a, e in zip(starts[:-1], starts[1:]):
        if e > a:
            ys = L.short_conv(x[:, a:e].contiguous(), w)
            dxs, _ = L.short_conv_bwd(x[:, a:e].contiguous(), w, dy[:, a:e].contiguous())
            torch.cuda.synchronize()
            assert torch.equal(ys, y[:, a:e]) and torch.equal(dxs, dx[:, a:e]), (a, e)


def test_short_conv_empty_and_deterministic():
    L = lrt()
    x = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((64, 4), generator=gen(3), device="cuda")
    y = L.short_conv(x, w)
    dx, dw = L.short_conv_bwd(x, w, x)
    torch.cuda.synchronize()
    assert y.numel() == 0 and dx.numel() == 0 and torch.count_nonzero(dw).item() == 0
    x, w, dy = conv_inputs(2, 333, 192, 4, torch.bfloat16, 30)
    a = L.short_conv_bwd(x, w, dy)
    b = L.short_conv_bwd(x, w, dy)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_short_conv_full_size_sampled_channels():
    """q, k and v of the 2048-token training shape (B=16, H=8, d=128) through
    one call as the 3 x 1024 columns of one tensor; the filter is per channel,
    so the oracle on a few channel slices checks them exactly."""
    L = lrt()
    B, T, D, W = 16, 2048, 3 * 1024, 4
    say("[conv] full size [16, 2048, 3072] bf16")
    x, w, dy = conv_inputs(B, T, D, W, torch.bfloat16, 40)
    y = L.short_conv(x, w)
    dx, dw = L.short_conv_bwd(x, w, dy)
    torch.cuda.synchronize()
    for c0 in (0, 1020, D - 8):
        sl = slice(c0, c0 + 8)
        xs, ws, dys = x[..., sl].contiguous(), w[sl].contiguous(), dy[..., sl].contiguous()
        ry = cn.short_conv(xs, ws)
        rdx, rdw = cn.short_conv_bwd(xs, ws, dys)
        errs = (rel(f64(y[..., sl]), ry), rel(f64(dx[..., sl]), rdx), rel(f64(dw[sl]), rdw))
        say(f"  channels {c0}..{c0 + 7}: y={errs[0]:.2e} dx={errs[1]:.2e} dw={errs[2]:.2e}")
        assert max(errs) <= TOL[torch.bfloat16], errs


NORM = [
    # name, shape (.., d), dtype
    ("fp32_d16", (2, 37, 3, 16), torch.float32),
    ("fp32_d128", (3, 50, 2, 128), torch.float32),
    ("fp32_d256", (1, 7, 5, 256), torch.float32),
    ("bf16_d32", (2, 11, 4, 32), torch.bfloat16),
    ("bf16_d64", (1, 333, 2, 64), torch.bfloat16),
    ("bf16_d128", (2, 257, 8, 128), torch.bfloat16),
    ("bf16_d256", (1, 3, 1, 256), torch.bfloat16),
]


def norm_inputs(shape, dt, seed):
    d = shape[-1]
    o = torch.randn(shape, generator=gen(seed), device="cuda").to(dt)
    z = torch.randn(shape, generator=gen(seed + 1), device="cuda").to(dt)
    w = 1.0 + 0.1 * torch.randn((d,), generator=gen(seed + 2), device="cuda")
    dy = torch.randn(shape, generator=gen(seed + 3), device="cuda").to(dt)
    return o, z, w, dy


@pytest.mark.parametrize("case", NORM, ids=[c[0] for c in NORM])
def test_gated_rmsnorm(case):
    name, shape, dt = case
    say(f"[gated norm] {name}")
    L = lrt()
    o, z, w, dy = norm_inputs(shape, dt, 50)
    y = L.gated_rmsnorm(o, z, w)
    do, dz, dw = L.gated_rmsnorm_bwd(o, z, w, dy)
    torch.cuda.synchronize()
    ry = cn.gated_rmsnorm(o, z, w)
    rdo, rdz, rdw = cn.gated_rmsnorm_bwd(o, z, w, dy)
    errs = {"y": rel(f64(y), ry), "do": rel(f64(do), rdo), "dz": rel(f64(dz), rdz), "dw": rel(f64(dw), rdw)}
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if v > TOL[dt]}
    assert not bad, bad


def test_gated_rmsnorm_empty_deterministic_and_full_size():
    L = lrt()
    o = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((128,), device="cuda")
    y = L.gated_rmsnorm(o, o, w)
    do, dz, dw = L.gated_rmsnorm_bwd(o, o, w, o)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.count_nonzero(dw).item() == 0
    # the mixer output of the 2048-token training shape, B = 16, H = 8, d_v = 128
    say("[gated norm] full size [16, 2048, 8, 128] bf16")
    o, z, w, dy = norm_inputs((16, 2048, 8, 128), torch.bfloat16, 60)
    a = L.gated_rmsnorm_bwd(o, z, w, dy)
    b = L.gated_rmsnorm_bwd(o, z, w, dy)
    y = L.gated_rmsnorm(o, z, w)
    torch.cuda.synchronize()
    for x1, x2 in zip(a, b):
        assert torch.equal(x1, x2)
    rows = slice(0, 2)  # every element of two batch rows; dw over all rows
    ry = cn.gated_rmsnorm(o[rows], z[rows], w)
    rdo, rdz, _ = cn.gated_rmsnorm_bwd(o[rows], z[rows], w, dy[rows])
    _, _, rdw = cn.gated_rmsnorm_bwd(o, z, w, dy)
    errs = (rel(f64(y[rows]), ry), rel(f64(a[0][rows]), rdo), rel(f64(a[1][rows]), rdz), rel(f64(a[2]), rdw))
    say("  y={:.2e} do={:.2e} dz={:.2e} dw={:.2e}".format(*errs))
    assert max(errs) <= TOL[torch.bfloat16], errs
