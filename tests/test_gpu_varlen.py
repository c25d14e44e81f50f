"""GPU parity of the packed variable-length entry points (gdn_fwd_varlen,
kda_fwd_varlen, gdn_bwd_varlen) through the C ABI.

Packing is how the 1M-context guide for the 7-MLA / 21-GDN hybrid feeds
its GDN layers (20-160 sequences per 1M tokens): many sequences share one
[1, T, H, d] tensor and every sequence starts from its own initial state.
Each sequence's outputs must equal the dense entry point run on that
sequence alone -- bitwise, since the chunks restart at every sequence start
and the per-chunk arithmetic is the same -- and the fp64 oracle run on that
sequence, at the dtype's bar (1e-4 fp32, 1e-2 bf16).  Lengths include
sequences shorter than a chunk, a one-token sequence and an empty one.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_token_amd import synth

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def packed_inputs(op, lens, H, dk, dv, dt, gate, shift, seed):
    T = int(sum(lens))
    n = len(lens)
    inp = synth.make_inputs(op, 1, T, H, dk, dv, dtype=dt, seed=seed, device="cuda", gate=gate, gate_shift=shift,
                            h0_std=0.0, with_do=True)
    h0 = synth.randn((n, H, dk, dv), seed, "h0", "cuda", std=0.1)
    dht = synth.randn((n, H, dk, dv), seed, "dht", "cuda", std=0.1)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    return inp, h0, dht, cu


def seq(x, a, b):
    return None if x is None else x[:, a:b].contiguous()


FWD = [
    # op, lengths, H, d_k, d_v, chunk, dtype, gate, gate_shift
    ("gdn", [130, 7, 64, 1, 300, 0, 65], 2, 128, 128, 64, torch.bfloat16, "scalar", -2.0),
    ("gdn", [50, 16, 3, 97], 3, 64, 32, 16, torch.float32, "scalar", -6.0),
    ("kda", [130, 7, 64, 1, 200, 0, 65], 2, 128, 128, 64, torch.bfloat16, "perdim", 0.0),
    ("kda", [50, 16, 3, 97], 2, 64, 64, 32, torch.float32, "perdim", -2.0),
]


@pytest.mark.parametrize("case", FWD, ids=[f"{c[0]}_{len(c[1])}seq_C{c[5]}_{str(c[6])[6:]}" for c in FWD])
def test_varlen_forward(case):
    import linear_recurrent_token_amd as L
    op, lens, H, dk, dv, chunk, dt, gate, shift = case
    say(f"[varlen] fwd {case}")
    inp, h0, _, cu = packed_inputs(f"{op}_fwd", lens, H, dk, dv, dt, gate, shift, seed=11)
    q, k, v, la, beta = (inp[n] for n in ("q", "k", "v", "log_a", "beta"))
    fv = L.gdn_fwd_varlen if op == "gdn" else L.kda_fwd_varlen
    fd = L.gdn_fwd if op == "gdn" else L.kda_fwd
    o, ht = fv(q, k, v, la, beta, cu, h0, chunk=chunk)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(lens)])
    errs = []
    for s, (a, b) in enumerate(zip(starts[:-1], starts[1:])):
        hs = h0[s:s + 1].contiguous()
        od, hd = fd(seq(q, a, b), seq(k, a, b), seq(v, a, b), seq(la, a, b), seq(beta, a, b), hs, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], od), (s, a, b)
        assert torch.equal(ht[s:s + 1], hd), (s, a, b)
        if b > a:
            c = lambda x: None if x is None else x.cpu()
            ro, rh = oracle.fwd(op, c(seq(q, a, b)), c(seq(k, a, b)), c(seq(v, a, b)), c(seq(la, a, b)),
                                c(seq(beta, a, b)), c(hs))
            errs.append((rel(o[:, a:b].float().cpu().numpy(), ro), rel(ht[s:s + 1].cpu().numpy(), rh)))
    worst = np.max(np.array(errs), axis=0)
    say(f"  worst per-sequence rel err o={worst[0]:.2e} ht={worst[1]:.2e}")
    assert worst[0] <= TOL[dt] and worst[1] <= TOL[dt], worst


BWD = [
    # lengths, H, d_k, d_v, chunk, dtype, gate_shift
    ([130, 7, 64, 1, 300, 0, 65], 2, 128, 128, 64, torch.bfloat16, -2.0),
    ([50, 16, 3, 97], 2, 64, 32, 16, torch.float32, -6.0),
]


@pytest.mark.parametrize("case", BWD, ids=[f"{len(c[0])}seq_C{c[4]}_{str(c[5])[6:]}" for c in BWD])
def test_varlen_backward(case):
    import linear_recurrent_token_amd as L
    lens, H, dk, dv, chunk, dt, shift = case
    say(f"[varlen] bwd {case}")
    inp, h0, dht, cu = packed_inputs("gdn_fwd_bwd", lens, H, dk, dv, dt, "scalar", shift, seed=12)
    q, k, v, la, beta, do = (inp[n] for n in ("q", "k", "v", "log_a", "beta", "do"))
    g = L.gdn_bwd_varlen(q, k, v, la, beta, cu, h0, do, dht, chunk=chunk)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(lens)])
    names = ("dq", "dk", "dv", "dlog_a", "dbeta", "dh0")
    worst = {n: 0.0 for n in names}
    for s, (a, b) in enumerate(zip(starts[:-1], starts[1:])):
        hs, ds = h0[s:s + 1].contiguous(), dht[s:s + 1].contiguous()
        gd = L.gdn_bwd(seq(q, a, b), seq(k, a, b), seq(v, a, b), seq(la, a, b), seq(beta, a, b), hs, seq(do, a, b),
                       ds, chunk=chunk)
        torch.cuda.synchronize()
        for name, x, y in zip(names, g, gd):
            part = x[s:s + 1] if name == "dh0" else x[:, a:b]
            assert torch.equal(part, y), (name, s, a, b)
        if b > a:
            c = lambda x: None if x is None else x.cpu()
            ref = oracle.bwd("gdn", c(seq(q, a, b)), c(seq(k, a, b)), c(seq(v, a, b)), c(seq(la, a, b)),
                             c(seq(beta, a, b)), c(hs), c(seq(do, a, b)), c(ds))
            for name, x, r in zip(names, g, ref):
                part = x[s:s + 1] if name == "dh0" else x[:, a:b]
                worst[name] = max(worst[name], rel(part.float().cpu().numpy(), r))
    say("  worst per-sequence " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))
    bad = {n: e for n, e in worst.items() if e > TOL[dt]}
    assert not bad, bad
