"""The torch.autograd bindings (linear_recurrent_token_amd.autograd): the
gradients autograd hands back are exactly those of the library's training
pair (*_fwd_train + *_bwd_saved) for the same upstream gradients (bitwise),
and the pieces compose
(short conv -> mixer -> gated norm) into one differentiable layer."""
import sys

import pytest
import torch

from linear_recurrent_token_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def leaf(t):
    return None if t is None else t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("op", ["gdn", "kda", "ssd"])
@pytest.mark.parametrize("with_h0", [False, True])
def test_mixer_autograd_equals_backward_entry(op, with_h0):
    import linear_recurrent_token_amd as L
    from linear_recurrent_token_amd import autograd as A
    say(f"[autograd] {op} h0={with_h0}")
    inp = synth.make_inputs(f"{op}_fwd_bwd", 2, 150, 2, 64, 64, dtype=torch.bfloat16, seed=7, device="cuda",
                            gate="perdim" if op == "kda" else "scalar", h0_std=0.1 if with_h0 else 0.0,
                            dht_std=0.1)
    q, k, v, la, beta, h0 = (leaf(inp.get(n)) for n in ("q", "k", "v", "log_a", "beta", "h0"))
    do, dht = inp["do"], inp["dht"]
    det = lambda t: None if t is None else t.detach()
    # the reference: the same training pair called directly
    if op == "gdn":
        o, ht = A.gated_delta_net(q, k, v, la, beta, h0, chunk=32)
        args = (det(q), det(k), det(v), det(la), det(beta), det(h0))
        _, _, saved = L.gdn_fwd_train(*args, chunk=32)
        ref = L.gdn_bwd_saved(*args, do, saved, dht, chunk=32)
        ins = (q, k, v, la, beta, h0)
    elif op == "kda":
        o, ht = A.kimi_delta_attention(q, k, v, la, beta, h0, chunk=32)
        args = (det(q), det(k), det(v), det(la), det(beta), det(h0))
        _, _, saved = L.kda_fwd_train(*args, chunk=32)
        ref = L.kda_bwd_saved(*args, do, saved, dht, chunk=32)
        ins = (q, k, v, la, beta, h0)
    else:
        o, ht = A.mamba2(q, k, v, la, h0, chunk=32)
        args = (det(q), det(k), det(v), det(la), det(h0))
        _, _, saved = L.ssd_fwd_train(*args, chunk=32)
        ref = L.ssd_bwd_saved(*args, do, saved, dht, chunk=32)
        ins = (q, k, v, la, h0)
    want = [t for t in ins if t is not None]
    got = torch.autograd.grad((o, ht), want, (do, dht))
    ref = [r for r, t in zip(ref, ins) if t is not None]
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert g.dtype == r.dtype and torch.equal(g, r)


def test_conv_and_norm_autograd_equal_backward_entries():
    import linear_recurrent_token_amd as L
    from linear_recurrent_token_amd import autograd as A
    g = torch.Generator(device="cuda").manual_seed(3)
    x = leaf(torch.randn((2, 70, 96), generator=g, device="cuda").to(torch.bfloat16))
    w = leaf(0.5 * torch.randn((96, 4), generator=g, device="cuda"))
    dy = torch.randn((2, 70, 96), generator=g, device="cuda").to(torch.bfloat16)
    y = A.short_conv(x, w)
    gx, gw = torch.autograd.grad(y, (x, w), dy)
    rx, rw = L.short_conv_bwd(x.detach(), w.detach(), dy)
    assert torch.equal(y, L.short_conv(x.detach(), w.detach()))
    assert torch.equal(gx, rx) and torch.equal(gw, rw)
    o = leaf(torch.randn((2, 70, 3, 128), generator=g, device="cuda").to(torch.bfloat16))
    z = leaf(torch.randn((2, 70, 3, 128), generator=g, device="cuda").to(torch.bfloat16))
    wn = leaf(1 + 0.1 * torch.randn((128,), generator=g, device="cuda"))
    dn = torch.randn((2, 70, 3, 128), generator=g, device="cuda").to(torch.bfloat16)
    yn = A.gated_rms_norm(o, z, wn)
    go, gz, gwn = torch.autograd.grad(yn, (o, z, wn), dn)
    ro, rz, rwn = L.gated_rmsnorm_bwd(o.detach(), z.detach(), wn.detach(), dn)
    torch.cuda.synchronize()
    assert torch.equal(go, ro) and torch.equal(gz, rz) and torch.equal(gwn, rwn)


def test_layer_composes():
    """x -> short conv -> q, k (L2-normalised), v -> Gated DeltaNet -> gated
    norm -> loss: one backward reaches every parameter with finite values."""
    from linear_recurrent_token_amd import autograd as A
    B, T, H, d = 2, 130, 2, 64
    g = torch.Generator(device="cuda").manual_seed(5)
    x = leaf(torch.randn((B, T, 3 * H * d), generator=g, device="cuda").to(torch.bfloat16))
    wc = leaf(0.5 * torch.randn((3 * H * d, 4), generator=g, device="cuda"))
    la = leaf(-torch.nn.functional.softplus(torch.randn((B, T, H), generator=g, device="cuda")))
    beta = leaf(torch.sigmoid(torch.randn((B, T, H), generator=g, device="cuda")))
    zg = leaf(torch.randn((B, T, H, d), generator=g, device="cuda").to(torch.bfloat16))
    wn = leaf(torch.ones((d,), device="cuda"))
    y = A.short_conv(x, wc).view(B, T, 3, H, d)
    q = torch.nn.functional.normalize(y[:, :, 0].float(), dim=-1).to(torch.bfloat16).contiguous()
    k = torch.nn.functional.normalize(y[:, :, 1].float(), dim=-1).to(torch.bfloat16).contiguous()
    v = y[:, :, 2].contiguous()
    o, _ = A.gated_delta_net(q, k, v, la, beta, chunk=64)
    out = A.gated_rms_norm(o, zg, wn)
    loss = out.float().pow(2).mean()
    loss.backward()
    torch.cuda.synchronize()
    for name, t in (("x", x), ("wc", wc), ("log_a", la), ("beta", beta), ("z", zg), ("w_norm", wn)):
        assert t.grad is not None and torch.isfinite(t.grad.float()).all(), name
        assert t.grad.float().abs().max() > 0, name
