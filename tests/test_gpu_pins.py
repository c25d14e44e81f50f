"""GPU parity on the cases the named workloads do not reach, through the C ABI:

* exact retrieval: no decay (log a = 0), beta = 1 and orthonormal keys, so
  every stored value is read back exactly by its key, whatever the initial
  state (the delta rule's defining property, Gated DeltaNet and Kimi Delta
  Attention in the mixer list under Table 2 of the AMD ROCm blog "Pretraining
  hybrid LLMs with Primus");
* bitwise determinism of every backward (the gate and beta gradients are
  reductions over tokens and dimensions, summed in a fixed order);
* state chaining of two calls for every mixer and dtype;
* the segment-parallel forward scan in fp32 at the fp32 bar, with slow gates,
  small beta and a unit-scale initial state (the carried state dominates).

Bar: max|got - oracle| / max|oracle| per tensor <= 1e-4 (fp32), 1e-2 (bf16).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_token_amd import synth

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
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def cpu(x):
    return None if x is None else x.detach().cpu()


def fwd(L, op, q, k, v, la, beta, h0, chunk):
    if op == "gdn":
        return L.gdn_fwd(q, k, v, la, beta, h0, chunk=chunk)
    if op == "kda":
        return L.kda_fwd(q, k, v, la, beta, h0, chunk=chunk)
    return L.ssd_fwd(q, k, v, la, h0, chunk=chunk)


RETRIEVAL = [
    # op, B, T, H, d_k, d_v, chunk, dtype
    ("gdn", 2, 128, 2, 128, 128, 64, torch.float32),
    ("gdn", 2, 128, 2, 128, 128, 64, torch.bfloat16),
    ("gdn", 1, 61, 3, 64, 32, 16, torch.float32),
    ("gdn", 1, 100, 2, 128, 64, 32, torch.bfloat16),
    ("kda", 2, 128, 2, 128, 128, 64, torch.bfloat16),
    ("kda", 1, 61, 2, 64, 64, 16, torch.float32),
    ("kda", 1, 100, 2, 128, 64, 32, torch.bfloat16),
]


@pytest.mark.parametrize("case", RETRIEVAL, ids=[f"{c[0]}_T{c[2]}_C{c[6]}_{str(c[7])[6:]}" for c in RETRIEVAL])
def test_exact_retrieval(case):
    """a = 1, beta = 1, orthonormal keys, h0 ~ N(0, 1): H_T^T k_j = v_j for
    every stored key and o_t = v_j(t) for q_t = k_j(t), j(t) <= t."""
    op, B, T, H, dk, dv, chunk, dt = case
    L = lrt()
    say(f"[pins] retrieval {case}")
    inp = synth.make_inputs(f"{op}_fwd", B, T, H, dk, dv, dtype=dt, seed=3, device="cuda", gate="zero",
                            beta_kind="one", keys="orthonormal", h0_std=1.0)
    q, k, v, la, beta, h0 = (inp[n] for n in ("q", "k", "v", "log_a", "beta", "h0"))
    o, ht = fwd(L, op, q, k, v, la, beta, h0, chunk)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd(op, cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0))
    eo, eh = rel(o.float().cpu().numpy(), ro), rel(ht.cpu().numpy(), rh)
    say(f"  vs oracle o={eo:.2e} ht={eh:.2e}")
    assert eo <= TOL[dt] and eh <= TOL[dt], (eo, eh)
    # the property itself: the values come back (fp32 keys are orthonormal to
    # about 1e-7; bf16 keys only to bf16 rounding, so only parity is exact there)
    vv = v.double().cpu().numpy()
    idx = inp["qidx"].cpu().numpy()
    want = np.take_along_axis(vv, np.repeat(idx[..., None], dv, -1), 1)
    back = np.einsum("bhde,bthd->bthe", ht.double().cpu().numpy(), k.double().cpu().numpy())
    tol = 1e-4 if dt == torch.float32 else 5e-2
    er, eb = rel(o.double().cpu().numpy(), want), rel(back, vv)
    say(f"  retrieval o={er:.2e} H^T k={eb:.2e}")
    assert er <= tol and eb <= tol, (er, eb)


def _grads(L, variant, inp, chunk, saved=None):
    q, k, v, la, beta, h0, do, dht = (inp.get(n) for n in ("q", "k", "v", "log_a", "beta", "h0", "do", "dht"))
    if variant == "gdn":
        if saved is not None:
            return L.gdn_bwd_saved(q, k, v, la, beta, h0, do, saved, dht, chunk=chunk)
        return L.gdn_bwd(q, k, v, la, beta, h0, do, dht, chunk=chunk)
    if saved is not None:
        return L.ssd_bwd_saved(q, k, v, la, h0, do, saved, dht, chunk=chunk)
    return L.ssd_bwd(q, k, v, la, h0, do, dht, chunk=chunk)


DET = [
    # variant, B, T, H, d, chunk, dtype
    ("gdn", 2, 300, 2, 128, 64, torch.bfloat16),
    ("gdn", 1, 77, 2, 64, 32, torch.float32),
    ("ssd", 2, 300, 2, 128, 64, torch.bfloat16),
    ("ssd", 1, 77, 2, 64, 16, torch.float32),
]


@pytest.mark.parametrize("case", DET, ids=[f"{c[0]}_d{c[4]}_C{c[5]}_{str(c[6])[6:]}" for c in DET])
def test_bwd_bitwise_deterministic(case):
    """Two backward calls on the same inputs give bitwise-identical gradients,
    through the stateless and the saved pair."""
    variant, B, T, H, d, chunk, dt = case
    L = lrt()
    say(f"[pins] determinism {case}")
    inp = synth.make_inputs(f"{variant}_fwd_bwd", B, T, H, d, d, dtype=dt, seed=4, device="cuda",
                            gate_shift=-2.0, h0_std=0.1, dht_std=0.1)
    a = _grads(L, variant, inp, chunk)
    b = _grads(L, variant, inp, chunk)
    if variant == "gdn":
        _, _, saved = L.gdn_fwd_train(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["h0"], chunk=chunk)
    else:
        _, _, saved = L.ssd_fwd_train(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["h0"], chunk=chunk)
    c = _grads(L, variant, inp, chunk, saved)
    d2 = _grads(L, variant, inp, chunk, saved)
    torch.cuda.synchronize()
    for x, y, z, w in zip(a, b, c, d2):
        if x is None:
            continue
        assert torch.equal(x, y)
        assert torch.equal(z, w)


CHAIN = [
    # op, dtype, d_k, d_v, chunk, split points
    ("gdn", torch.bfloat16, 128, 128, 64, (128, 77)),
    ("ssd", torch.float32, 64, 64, 32, (64, 77)),
    ("ssd", torch.bfloat16, 128, 128, 64, (128, 77)),
    ("kda", torch.float32, 64, 64, 32, (64, 77)),
    ("kda", torch.bfloat16, 128, 128, 64, (128, 77)),
]


@pytest.mark.parametrize("case", CHAIN, ids=[f"{c[0]}_{str(c[1])[6:]}" for c in CHAIN])
def test_state_chaining(case):
    """fwd(x[:t1]) -> ht, then fwd(x[t1:], h0 = ht): o and the final state
    match the oracle's one-call result at the dtype's bar; a split on a chunk
    boundary reproduces the one-call result bitwise (the same operations in
    the same order)."""
    op, dt, dk, dv, chunk, splits = case
    L = lrt()
    say(f"[pins] chaining {case}")
    gate = "perdim" if op == "kda" else "scalar"
    inp = synth.make_inputs(f"{op}_fwd", 2, 300, 2, dk, dv, dtype=dt, seed=5, device="cuda", gate=gate,
                            gate_shift=-6.0, h0_std=0.1)
    q, k, v, la, beta, h0 = (inp.get(n) for n in ("q", "k", "v", "log_a", "beta", "h0"))
    o, ht = fwd(L, op, q, k, v, la, beta, h0, chunk)
    ro, rh = oracle.fwd(op, cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0))

    def part(x, a, b):
        return None if x is None else x[:, a:b].contiguous()

    for t1 in splits:
        oa, ha = fwd(L, op, part(q, 0, t1), part(k, 0, t1), part(v, 0, t1), part(la, 0, t1), part(beta, 0, t1), h0,
                     chunk)
        ob, hb = fwd(L, op, part(q, t1, 300), part(k, t1, 300), part(v, t1, 300), part(la, t1, 300),
                     part(beta, t1, 300), ha, chunk)
        torch.cuda.synchronize()
        oc = torch.cat([oa, ob], 1)
        eo, eh = rel(oc.float().cpu().numpy(), ro), rel(hb.cpu().numpy(), rh)
        say(f"  split {t1}: o={eo:.2e} ht={eh:.2e}")
        assert eo <= TOL[dt] and eh <= TOL[dt], (t1, eo, eh)
        if t1 % chunk == 0:
            assert torch.equal(oc, o) and torch.equal(hb, ht), t1


SEG_FP32 = [
    # op, T, H, d, chunk -- B * H small and many chunks: the forward scan runs
    # segment-parallel; fp32 operands throughout (the carry included)
    ("gdn", 4000, 2, 64, 32),
    ("gdn", 1500, 1, 32, 16),
    ("kda", 4000, 2, 64, 32),
]


@pytest.mark.parametrize("case", SEG_FP32, ids=[f"{c[0]}_T{c[1]}_d{c[3]}" for c in SEG_FP32])
def test_fp32_segmented_scan(case):
    op, T, H, d, chunk = case
    L = lrt()
    say(f"[pins] fp32 segmented {case}")
    gate = "perdim" if op == "kda" else "scalar"
    inp = synth.make_inputs(f"{op}_fwd", 1, T, H, d, d, dtype=torch.float32, seed=6, device="cuda", gate=gate,
                            gate_shift=-6.0, beta_shift=-4.0, h0_std=1.0)
    q, k, v, la, beta, h0 = (inp[n] for n in ("q", "k", "v", "log_a", "beta", "h0"))
    o, ht = fwd(L, op, q, k, v, la, beta, h0, chunk)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd(op, cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0))
    eo, eh = rel(o.cpu().numpy(), ro), rel(ht.cpu().numpy(), rh)
    say(f"  o={eo:.2e} ht={eh:.2e}")
    assert eo <= 1e-4 and eh <= 1e-4, (eo, eh)
    if op == "gdn":
        # the training forward takes the same segmented scan (saving states)
        o2, ht2, _ = L.gdn_fwd_train(q, k, v, la, beta, h0, chunk=chunk)
        torch.cuda.synchronize()
        eo2, eh2 = rel(o2.cpu().numpy(), ro), rel(ht2.cpu().numpy(), rh)
        say(f"  train fwd o={eo2:.2e} ht={eh2:.2e}")
        assert eo2 <= 1e-4 and eh2 <= 1e-4, (eo2, eh2)
