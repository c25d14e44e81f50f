"""GPU parity of gdn_bwd and ssd_bwd against the fp64 oracle's
back-propagation through time, through the C ABI.

Bar: max|got - oracle| / max|oracle| per gradient tensor (dq, dk, dv,
dlog_a, dbeta (GDN only), dh0) <= 1e-4 for fp32 inputs and <= 1e-2 for bf16
inputs.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_token_amd import synth

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
NAMES = ("dq", "dk", "dv", "dlog_a", "dbeta", "dh0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def cpu(x):
    return None if x is None else x.detach().cpu()


def check_bwd(inp, chunk, tol, variant="gdn"):
    import linear_recurrent_token_amd as L
    q, k, v, la, beta, h0, do, dht = (inp.get(n) for n in ("q", "k", "v", "log_a", "beta", "h0", "do", "dht"))
    if variant == "gdn":
        got = L.gdn_bwd(q, k, v, la, beta, h0, do, dht, chunk=chunk)
        names = NAMES
    else:
        got = L.ssd_bwd(q, k, v, la, h0, do, dht, chunk=chunk)
        names = tuple(n for n in NAMES if n != "dbeta")
    torch.cuda.synchronize()
    ref = oracle.bwd(variant, cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0), cpu(do), cpu(dht))
    ref = [r for n, r in zip(NAMES, ref) if n in names]
    errs = {}
    for name, g, r in zip(names, got, ref):
        g = g.float().cpu().numpy()
        assert np.all(np.isfinite(g)), name
        errs[name] = rel(g, r)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if e > tol}
    assert not bad, bad


CASES = [
    # name, B, T, H, dk, dv, chunk, dtype, gate_shift, h0_std, dht_std
    ("fp32_tiny_cfg", 1, 64, 2, 16, 16, 16, torch.float32, 0.0, 0.0, 0.0),
    ("fp32_slow_h0_dht", 2, 77, 2, 32, 64, 32, torch.float32, -6.0, 0.1, 0.1),
    ("fp32_d64_C16", 1, 100, 2, 64, 64, 16, torch.float32, -6.0, 0.1, 0.1),
    ("bf16_slow_T61_C16", 2, 61, 3, 64, 64, 16, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_slow_C32", 1, 200, 2, 128, 128, 32, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_slow_C64", 2, 300, 2, 128, 128, 64, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_fast_C64", 2, 256, 2, 128, 128, 64, torch.bfloat16, 2.0, 0.1, 0.0),
    ("bf16_d16_dv32", 1, 100, 2, 16, 32, 16, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_dk32_dv128", 1, 100, 2, 32, 128, 32, torch.bfloat16, -6.0, 0.1, 0.1),
    # long sequence, slow gates: the state carry spans 64 chunks both ways
    ("bf16_long_slow_C64", 1, 4096 - 7, 2, 128, 128, 64, torch.bfloat16, -6.0, 0.1, 0.1),
    # fp32 at d = 128 with chunk 64 requested (the kernels run 16-token chunks,
    # the largest whose fp32 operands fit in LDS), and at d = 64, chunk 64
    ("fp32_d128_C64", 1, 150, 2, 128, 128, 64, torch.float32, -6.0, 0.1, 0.1),
    ("fp32_dk128_dv64_C64", 1, 100, 2, 128, 64, 64, torch.float32, -2.0, 0.1, 0.1),
    ("fp32_d64_C64", 2, 130, 2, 64, 64, 64, torch.float32, -6.0, 0.1, 0.1),
    # bf16 layouts of the gradient kernel: one d_k tile per wave at chunk 16
    # (the shared-fragment products), the dk rows over S^T with dT^T over the
    # dv rows (d = 64), neither (d_k 128, d_v 64), and a one-tile d_k
    ("bf16_d128_C16", 1, 90, 2, 128, 128, 16, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_d64_C64", 2, 130, 2, 64, 64, 64, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_dk128_dv64_C64", 1, 100, 2, 128, 64, 64, torch.bfloat16, -2.0, 0.1, 0.1),
    ("bf16_dk16_dv128_C64", 1, 100, 2, 16, 128, 64, torch.bfloat16, -6.0, 0.1, 0.1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_small(case):
    name, B, T, H, dk, dv, chunk, dt, shift, h0s, dhs = case
    say(f"[bwd] {name}")
    inp = synth.make_inputs("gdn_fwd_bwd", B, T, H, dk, dv, dtype=dt, seed=0, device="cuda",
                            gate_shift=shift, h0_std=h0s, dht_std=dhs)
    check_bwd(inp, chunk, TOL[dt])


def test_bwd_training_step_workload():
    """The Gated DeltaNet training-step workload at full size (B=16, T=2048,
    H=8, d=128, chunk 64, bf16), every gradient element against the oracle."""
    say("[bwd] workload gdn_train_bf16_2k")
    inp = synth.config_inputs("gdn_train_bf16_2k", device="cuda")
    check_bwd(inp, 64, TOL[torch.bfloat16])


SAVED_CASES = ["fp32_tiny_cfg", "fp32_slow_h0_dht", "bf16_slow_T61_C16", "bf16_slow_C32", "bf16_slow_C64",
               "bf16_d16_dv32", "bf16_long_slow_C64", "fp32_d128_C64", "fp32_d64_C64"]


@pytest.mark.parametrize("name", SAVED_CASES)
def test_fwd_train_and_bwd_saved(name):
    """gdn_fwd_train's outputs and gdn_bwd_saved's gradients against the
    oracle; a second gdn_bwd_saved on the same saved workspace (another
    upstream gradient) matches the stateless gdn_bwd for it.  The long case
    runs the segment-parallel forward scan (B*H small), whose saved states
    come from the segments' true starts."""
    import linear_recurrent_token_amd as L
    case = next(c for c in CASES if c[0] == name)
    _, B, T, H, dk, dv, chunk, dt, shift, h0s, dhs = case
    say(f"[fwd_train/bwd_saved] {name}")
    inp = synth.make_inputs("gdn_fwd_bwd", B, T, H, dk, dv, dtype=dt, seed=0, device="cuda",
                            gate_shift=shift, h0_std=h0s, dht_std=dhs)
    q, k, v, la, beta, h0, do, dht = (inp.get(n) for n in ("q", "k", "v", "log_a", "beta", "h0", "do", "dht"))
    o, ht, saved = L.gdn_fwd_train(q, k, v, la, beta, h0, chunk=chunk)
    got = L.gdn_bwd_saved(q, k, v, la, beta, h0, do, saved, dht, chunk=chunk)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd("gdn", cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0))
    ref = oracle.bwd("gdn", cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0), cpu(do), cpu(dht))
    errs = {"o": rel(o.float().cpu().numpy(), ro), "ht": rel(ht.cpu().numpy(), rh)}
    for n, g, r in zip(NAMES, got, ref):
        g = g.float().cpu().numpy()
        assert np.all(np.isfinite(g)), n
        errs[n] = rel(g, r)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if e > TOL[dt]}
    assert not bad, bad
    # the saved tensors survive a backward: reuse them for another do
    do2 = (torch.randn(do.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(5))).to(dt)
    again = L.gdn_bwd_saved(q, k, v, la, beta, h0, do2, saved, dht, chunk=chunk)
    plain = L.gdn_bwd(q, k, v, la, beta, h0, do2, dht, chunk=chunk)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, again, plain):
        x, y = x.float().cpu().numpy(), y.float().cpu().numpy()
        assert rel(x, y) <= TOL[dt], (n, rel(x, y))


def test_fwd_train_and_bwd_saved_workload():
    """The training-step workload (B=16, T=2048, H=8, d=128, chunk 64,
    bf16) through gdn_fwd_train + gdn_bwd_saved, every element against the
    oracle."""
    import linear_recurrent_token_amd as L
    say("[fwd_train/bwd_saved] workload gdn_train_bf16_2k")
    inp = synth.config_inputs("gdn_train_bf16_2k", device="cuda")
    q, k, v, la, beta, h0, do, dht = (inp.get(n) for n in ("q", "k", "v", "log_a", "beta", "h0", "do", "dht"))
    o, ht, saved = L.gdn_fwd_train(q, k, v, la, beta, h0, chunk=64)
    got = L.gdn_bwd_saved(q, k, v, la, beta, h0, do, saved, dht, chunk=64)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd("gdn", cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0))
    ref = oracle.bwd("gdn", cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0), cpu(do), cpu(dht))
    errs = {"o": rel(o.float().cpu().numpy(), ro), "ht": rel(ht.cpu().numpy(), rh)}
    errs.update({n: rel(g.float().cpu().numpy(), r) for n, g, r in zip(NAMES, got, ref)})
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if e > TOL[torch.bfloat16]}
    assert not bad, bad


SSD_CASES = [
    # name, B, T, H, dk, dv, chunk, dtype, gate_shift, h0_std, dht_std
    ("fp32_tiny", 1, 64, 2, 16, 16, 16, torch.float32, 0.0, 0.0, 0.0),
    ("fp32_slow_h0_dht_T77_C32", 2, 77, 2, 32, 64, 32, torch.float32, -6.0, 0.1, 0.1),
    ("bf16_slow_T61_C16", 2, 61, 3, 64, 64, 16, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_slow_C32", 1, 200, 2, 128, 128, 32, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_slow_C64_T300", 2, 300, 2, 128, 128, 64, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_default_gates_C64", 2, 256, 2, 128, 128, 64, torch.bfloat16, 0.0, 0.0, 0.0),
    ("bf16_dk32_dv128", 1, 100, 2, 32, 128, 32, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_long_slow_C64", 1, 4096 - 7, 2, 128, 128, 64, torch.bfloat16, -6.0, 0.1, 0.1),
    ("fp32_d128_C64", 1, 150, 2, 128, 128, 64, torch.float32, -6.0, 0.1, 0.1),
    ("bf16_d128_C16", 1, 90, 2, 128, 128, 16, torch.bfloat16, -6.0, 0.1, 0.1),
    ("bf16_d64_C64", 2, 130, 2, 64, 64, 64, torch.bfloat16, -6.0, 0.1, 0.1),
]


@pytest.mark.parametrize("case", SSD_CASES, ids=[c[0] for c in SSD_CASES])
def test_ssd_bwd_small(case):
    name, B, T, H, dk, dv, chunk, dt, shift, h0s, dhs = case
    say(f"[ssd_bwd] {name}")
    inp = synth.make_inputs("ssd_fwd_bwd", B, T, H, dk, dv, dtype=dt, seed=0, device="cuda",
                            gate_shift=shift, h0_std=h0s, dht_std=dhs)
    check_bwd(inp, chunk, TOL[dt], variant="ssd")


def test_ssd_bwd_workload_shape():
    """Mamba2 training step at the 2048-token shape (B=16, T=2048, H=8,
    d=128, chunk 64, bf16, the Mamba2 forward workload's distributions), every
    gradient element against the oracle."""
    say("[ssd_bwd] workload ssd_train_bf16_2k")
    inp = synth.config_inputs("ssd_train_bf16_2k", device="cuda")
    check_bwd(inp, 64, TOL[torch.bfloat16], variant="ssd")


SSD_SAVED_CASES = ["fp32_tiny", "fp32_slow_h0_dht_T77_C32", "bf16_slow_T61_C16", "bf16_slow_C64_T300",
                   "bf16_dk32_dv128", "bf16_long_slow_C64", "fp32_d128_C64"]


@pytest.mark.parametrize("name", SSD_SAVED_CASES)
def test_ssd_fwd_train_and_bwd_saved(name):
    """ssd_fwd_train's outputs and ssd_bwd_saved's gradients against the
    oracle; a second ssd_bwd_saved on the same saved workspace matches the
    stateless ssd_bwd for another upstream gradient."""
    import linear_recurrent_token_amd as L
    case = next(c for c in SSD_CASES if c[0] == name)
    _, B, T, H, dk, dv, chunk, dt, shift, h0s, dhs = case
    say(f"[ssd_fwd_train/ssd_bwd_saved] {name}")
    inp = synth.make_inputs("ssd_fwd_bwd", B, T, H, dk, dv, dtype=dt, seed=0, device="cuda",
                            gate_shift=shift, h0_std=h0s, dht_std=dhs)
    q, k, v, la, h0, do, dht = (inp.get(n) for n in ("q", "k", "v", "log_a", "h0", "do", "dht"))
    o, ht, saved = L.ssd_fwd_train(q, k, v, la, h0, chunk=chunk)
    got = L.ssd_bwd_saved(q, k, v, la, h0, do, saved, dht, chunk=chunk)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd("ssd", cpu(q), cpu(k), cpu(v), cpu(la), None, cpu(h0))
    ref = oracle.bwd("ssd", cpu(q), cpu(k), cpu(v), cpu(la), None, cpu(h0), cpu(do), cpu(dht))
    names = tuple(n for n in NAMES if n != "dbeta")
    ref = [r for n, r in zip(NAMES, ref) if n != "dbeta"]
    errs = {"o": rel(o.float().cpu().numpy(), ro), "ht": rel(ht.cpu().numpy(), rh)}
    for n, g, r in zip(names, got, ref):
        g = g.float().cpu().numpy()
        assert np.all(np.isfinite(g)), n
        errs[n] = rel(g, r)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if e > TOL[dt]}
    assert not bad, bad
    do2 = (torch.randn(do.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(5))).to(dt)
    again = L.ssd_bwd_saved(q, k, v, la, h0, do2, saved, dht, chunk=chunk)
    plain = L.ssd_bwd(q, k, v, la, h0, do2, dht, chunk=chunk)
    torch.cuda.synchronize()
    for n, x, y in zip(names, again, plain):
        x, y = x.float().cpu().numpy(), y.float().cpu().numpy()
        assert rel(x, y) <= TOL[dt], (n, rel(x, y))


def test_ssd_fwd_train_and_bwd_saved_workload():
    """The Mamba2 training step at the 2048-token shape through the saved
    pair, every element against the oracle."""
    import linear_recurrent_token_amd as L
    say("[ssd_fwd_train/ssd_bwd_saved] workload ssd_train_bf16_2k")
    inp = synth.config_inputs("ssd_train_bf16_2k", device="cuda")
    q, k, v, la, h0, do, dht = (inp.get(n) for n in ("q", "k", "v", "log_a", "h0", "do", "dht"))
    o, ht, saved = L.ssd_fwd_train(q, k, v, la, h0, chunk=64)
    got = L.ssd_bwd_saved(q, k, v, la, h0, do, saved, dht, chunk=64)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd("ssd", cpu(q), cpu(k), cpu(v), cpu(la), None, cpu(h0))
    ref = oracle.bwd("ssd", cpu(q), cpu(k), cpu(v), cpu(la), None, cpu(h0), cpu(do), cpu(dht))
    ref = [r for n, r in zip(NAMES, ref) if n != "dbeta"]
    errs = {"o": rel(o.float().cpu().numpy(), ro), "ht": rel(ht.cpu().numpy(), rh)}
    errs.update({n: rel(g.float().cpu().numpy(), r)
                 for n, g, r in zip(("dq", "dk", "dv", "dlog_a", "dh0"), got, ref)})
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if e > TOL[torch.bfloat16]}
    assert not bad, bad
