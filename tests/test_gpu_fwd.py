"""GPU parity of the forward mixers (gdn_fwd, ssd_fwd, kda_fwd) against the
fp64 CPU oracle, through the C ABI.

Bar: max|got - oracle| / max|oracle|, per output tensor, <= 1e-4 for fp32
inputs and <= 1e-2 for bf16 inputs.
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


def mixed_shift(T, H, chunk, device):
    """A gate shift per (token, head) that alternates by chunk: +3 (the
    chunk's decay far past e^60, the exact path) on chunks n with
    (n + h) % 3 == 0, -2 (the whole-chunk factorised path) elsewhere, so both
    paths and their interleaving over the chunks are exercised."""
    n = torch.arange(T, device=device).view(T, 1) // chunk
    h = torch.arange(H, device=device).view(1, H)
    return torch.where((n + h) % 3 == 0, 3.0, -2.0).view(1, T, H, 1)


def run_fwd(op, inp, chunk, cols=None):
    L = lrt()
    q, k, v, la = inp["q"], inp["k"], inp["v"], inp["log_a"]
    beta, h0 = inp.get("beta"), inp.get("h0")
    if op == "gdn":
        o, ht = L.gdn_fwd(q, k, v, la, beta, h0, chunk=chunk)
    elif op == "ssd":
        o, ht = L.ssd_fwd(q, k, v, la, h0, chunk=chunk)
    else:
        o, ht = L.kda_fwd(q, k, v, la, beta, h0, chunk=chunk)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd(op, cpu(q), cpu(k), cpu(v), cpu(la), cpu(beta), cpu(h0), cols=cols)
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    if cols is not None:
        o, ht = o[..., cols[0]:cols[0] + cols[1]], ht[..., cols[0]:cols[0] + cols[1]]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    return rel(o, ro), rel(ht, rh)


CASES = [
    # name, op, B, T, H, dk, dv, chunk, dtype, gate_shift, h0_std
    ("gdn_fp32_tiny_cfg", "gdn", 1, 64, 2, 16, 16, 16, torch.float32, 0.0, 0.0),
    ("gdn_fp32_slow_h0", "gdn", 2, 150, 2, 32, 64, 32, torch.float32, -6.0, 0.1),
    ("gdn_fp32_d128", "gdn", 1, 130, 2, 128, 128, 64, torch.float32, -6.0, 0.1),
    ("gdn_fp32_dk64_dv128_C64", "gdn", 2, 100, 2, 64, 128, 64, torch.float32, -2.0, 0.1),
    ("ssd_fp32_d128_C64", "ssd", 1, 130, 2, 128, 128, 64, torch.float32, -6.0, 0.1),
    ("gdn_bf16_slow_T61_C16", "gdn", 2, 61, 3, 64, 64, 16, torch.bfloat16, -6.0, 0.1),
    ("gdn_bf16_slow_C32", "gdn", 2, 200, 2, 128, 128, 32, torch.bfloat16, -6.0, 0.1),
    ("gdn_bf16_slow_C64", "gdn", 2, 300, 2, 128, 128, 64, torch.bfloat16, -6.0, 0.1),
    ("gdn_bf16_fast_C64", "gdn", 2, 256, 2, 128, 128, 64, torch.bfloat16, 2.0, 0.1),
    ("gdn_bf16_d16_dv32", "gdn", 1, 100, 2, 16, 32, 16, torch.bfloat16, -6.0, 0.1),
    ("gdn_bf16_dk32_dv128", "gdn", 1, 100, 2, 32, 128, 32, torch.bfloat16, -6.0, 0.1),
    ("ssd_fp32_slow", "ssd", 1, 97, 2, 32, 32, 16, torch.float32, -6.0, 0.1),
    ("ssd_bf16_slow_C64", "ssd", 2, 300, 2, 128, 128, 64, torch.bfloat16, -6.0, 0.1),
    ("ssd_bf16_fast_T2048", "ssd", 1, 2048, 2, 128, 128, 64, torch.bfloat16, 0.0, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_small(case):
    name, op, B, T, H, dk, dv, chunk, dt, shift, h0s = case
    say(f"[fwd] {name}")
    inp = synth.make_inputs(f"{op}_fwd", B, T, H, dk, dv, dtype=dt, seed=0, device="cuda",
                            gate_shift=shift, h0_std=h0s)
    eo, eh = run_fwd(op, inp, chunk)
    say(f"  rel err o={eo:.2e} ht={eh:.2e}")
    assert eo <= TOL[dt] and eh <= TOL[dt], (eo, eh)


@pytest.mark.parametrize("name,op", [("gdn_fp32_tiny", "gdn"), ("ssd_bf16_2k", "ssd"), ("gdn_bf16_2k", "gdn")])
def test_fwd_named_workloads(name, op):
    """The named workloads at full size, every element of o and ht against the
    oracle (about 3 s of fp64 work on 8 cores at the 2048-token shapes)."""
    say(f"[fwd] workload {name}")
    c = synth.CONFIGS[name]
    inp = synth.config_inputs(name, device="cuda")
    eo, eh = run_fwd(op, inp, c["chunk"])
    say(f"  rel err o={eo:.2e} ht={eh:.2e}")
    assert eo <= TOL[c["dtype"]] and eh <= TOL[c["dtype"]], (eo, eh)


def test_fwd_state_chaining():
    """Two calls with ht -> h0 equal one call (chunk-aligned and ragged splits)."""
    L = lrt()
    inp = synth.make_inputs("gdn_fwd", 1, 200, 2, 64, 64, dtype=torch.float32, device="cuda",
                            gate_shift=-6.0, h0_std=0.1)
    q, k, v, la, beta, h0 = (inp[n] for n in ("q", "k", "v", "log_a", "beta", "h0"))
    o, ht = L.gdn_fwd(q, k, v, la, beta, h0, chunk=32)
    for t1 in (64, 77):
        oa, ha = L.gdn_fwd(q[:, :t1].contiguous(), k[:, :t1].contiguous(), v[:, :t1].contiguous(),
                           la[:, :t1].contiguous(), beta[:, :t1].contiguous(), h0, chunk=32)
        ob, hb = L.gdn_fwd(q[:, t1:].contiguous(), k[:, t1:].contiguous(), v[:, t1:].contiguous(),
                           la[:, t1:].contiguous(), beta[:, t1:].contiguous(), ha, chunk=32)
        torch.cuda.synchronize()
        assert rel(torch.cat([oa, ob], 1).cpu(), o.cpu()) <= 1e-5
        assert rel(hb.cpu(), ht.cpu()) <= 1e-5


def test_fwd_empty_sequence_and_inplace_state():
    L = lrt()
    inp = synth.make_inputs("gdn_fwd", 2, 0, 2, 32, 32, dtype=torch.bfloat16, device="cuda", h0_std=0.1)
    o, ht = L.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["h0"], chunk=16)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(ht, inp["h0"])
    # ht aliasing h0: in-place carry
    inp = synth.make_inputs("gdn_fwd", 1, 40, 2, 32, 32, dtype=torch.bfloat16, device="cuda", h0_std=0.1)
    ref_o, ref_h = L.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["h0"], chunk=16)
    h = inp["h0"].clone()
    o2, _ = L.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], h, chunk=16, ht=h)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o) and torch.equal(h, ref_h)


def test_fwd_deterministic():
    L = lrt()
    inp = synth.make_inputs("gdn_fwd", 2, 333, 4, 128, 128, dtype=torch.bfloat16, device="cuda",
                            gate_shift=0.0, h0_std=0.1)
    a = L.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["h0"])
    b = L.gdn_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["h0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


KDA_CASES = [
    # name, B, T, H, dk, dv, chunk, dtype, gate kind, gate_shift, h0_std
    ("kda_fp32_perdim_C16", 1, 70, 2, 32, 32, 16, torch.float32, "perdim", 0.0, 0.1),
    ("kda_fp32_slow_C64", 1, 150, 2, 64, 64, 64, torch.float32, "perdim", -6.0, 0.1),
    ("kda_bf16_perdim_C64", 2, 200, 2, 128, 128, 64, torch.bfloat16, "perdim", 0.0, 0.1),
    ("kda_bf16_perdim_fast_C32", 1, 130, 2, 128, 128, 32, torch.bfloat16, "perdim", 2.0, 0.1),
    ("kda_bf16_slow_T61_C16", 2, 61, 2, 64, 32, 16, torch.bfloat16, "perdim", -6.0, 0.1),
    ("kda_bf16_lowrank_C64", 1, 256, 4, 128, 128, 64, torch.bfloat16, "lowrank", 0.0, 0.0),
    # fp32 at d = 128, chunk 64 requested (the kernels run 32-token chunks)
    ("kda_fp32_d128_C64", 1, 150, 2, 128, 128, 64, torch.float32, "perdim", -2.0, 0.1),
    ("kda_fp32_d64_C64", 1, 150, 2, 64, 64, 64, torch.float32, "perdim", 0.0, 0.1),
    # chunks on both paths, interleaved over heads and tokens
    ("kda_bf16_mixed_C64", 2, 443, 3, 128, 128, 64, torch.bfloat16, "perdim", "mixed", 0.1),
    ("kda_fp32_mixed_d64_C64", 1, 300, 3, 64, 64, 64, torch.float32, "perdim", "mixed", 0.1),
    ("kda_bf16_mixed_C16", 1, 150, 2, 32, 64, 16, torch.bfloat16, "perdim", "mixed", 0.1),
]


@pytest.mark.parametrize("case", KDA_CASES, ids=[c[0] for c in KDA_CASES])
def test_kda_fwd_small(case):
    name, B, T, H, dk, dv, chunk, dt, gate, shift, h0s = case
    say(f"[fwd] {name}")
    if shift == "mixed":
        shift = mixed_shift(T, H, chunk, "cuda")
    inp = synth.make_inputs("kda_fwd", B, T, H, dk, dv, dtype=dt, seed=0, device="cuda", gate=gate,
                            gate_shift=shift, h0_std=h0s)
    eo, eh = run_fwd("kda", inp, chunk)
    say(f"  rel err o={eo:.2e} ht={eh:.2e}")
    assert eo <= TOL[dt] and eh <= TOL[dt], (eo, eh)


def test_kda_uniform_gate_matches_gdn_kernel():
    """A per-dimension gate that is equal over d_k must give the GDN result."""
    L = lrt()
    inp = synth.make_inputs("gdn_fwd", 1, 200, 2, 128, 128, dtype=torch.bfloat16, device="cuda",
                            gate_shift=0.0, h0_std=0.1)
    q, k, v, la, beta, h0 = (inp[n] for n in ("q", "k", "v", "log_a", "beta", "h0"))
    og, hg = L.gdn_fwd(q, k, v, la, beta, h0)
    ok, hk = L.kda_fwd(q, k, v, la[..., None].expand(1, 200, 2, 128).contiguous(), beta, h0)
    torch.cuda.synchronize()
    assert rel(ok.float().cpu(), og.float().cpu()) <= 1e-2
    assert rel(hk.cpu(), hg.cpu()) <= 1e-2


def test_kda_long_context_workload():
    """KDA at B=1, H=16, T=2^20, d=128, chunk 64 (16,384 chunks per head, the
    state carried across all of them), rank-16 gate.  The whole forward runs on
    the GPU; the oracle checks the last 8 value columns of o and ht (columns of
    the state never mix, so the sample is exact for those columns)."""
    L = lrt()
    name = "kda_bf16_1m"
    say(f"[fwd] workload {name}")
    c = synth.CONFIGS[name]
    inp = synth.config_inputs(name, device="cuda")
    q, k, v, la, beta = (inp[n] for n in ("q", "k", "v", "log_a", "beta"))
    o, ht = L.kda_fwd(q, k, v, la, beta, None, chunk=c["chunk"])
    torch.cuda.synchronize()
    c0, nc = c["dv"] - 8, 8
    o_s = o[..., c0:c0 + nc].float().cpu().numpy()
    ht_s = ht[..., c0:c0 + nc].cpu().numpy()
    del o, ht
    say("  gpu done; oracle on 8 columns")
    ro, rh = oracle.fwd("kda", q.cpu(), k.cpu(), v.cpu(), la.cpu(), beta.cpu(), None, cols=(c0, nc))
    assert np.all(np.isfinite(o_s)) and np.all(np.isfinite(ht_s))
    eo, eh = rel(o_s, ro), rel(ht_s, rh)
    say(f"  rel err o={eo:.2e} ht={eh:.2e}")
    assert eo <= TOL[c["dtype"]] and eh <= TOL[c["dtype"]], (eo, eh)


SEG_CASES = [
    # name, op, B, T, H, dk, dv, chunk, gate kind, gate_shift, h0_std -- few (b, h) pairs and
    # long sequences: the forward scan runs segment-parallel (local pass, carry, scan)
    ("gdn_seg10_slow_h0", "gdn", 1, 10240 - 13, 1, 128, 128, 64, "scalar", -6.0, 0.1),
    ("gdn_seg2_fast", "gdn", 1, 2560, 2, 128, 128, 64, "scalar", 0.0, 0.1),
    ("kda_seg8_slow_C32", "kda", 1, 4096 - 5, 2, 64, 64, 32, "perdim", -6.0, 0.1),
    ("kda_seg4_perdim_C64", "kda", 1, 4096, 2, 128, 128, 64, "perdim", 0.0, 0.1),
    ("kda_seg4_lowrank_C64", "kda", 1, 4096, 2, 128, 128, 64, "lowrank", 0.0, 0.1),
    # fp32 through the segment carry (its MFMA in fp32), at the fp32 bar: slow
    # gates, small beta and a unit-scale h0, so the carried state dominates
    ("gdn_seg8_fp32_slow_C32", "gdn", 1, 4096 - 3, 2, 64, 64, 32, "scalar", -6.0, 1.0, torch.float32, -4.0),
    ("kda_seg8_fp32_slow_C32", "kda", 1, 4096 - 3, 2, 64, 64, 32, "perdim", -6.0, 1.0, torch.float32, -4.0),
]


@pytest.mark.parametrize("case", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_fwd_segmented_scan(case):
    name, op, B, T, H, dk, dv, chunk, gate, shift, h0s = case[:11]
    dt, bshift = case[11:] if len(case) > 11 else (torch.bfloat16, 0.0)
    say(f"[fwd] {name}")
    inp = synth.make_inputs(f"{op}_fwd", B, T, H, dk, dv, dtype=dt, seed=1, device="cuda", gate=gate,
                            gate_shift=shift, h0_std=h0s, beta_shift=bshift)
    eo, eh = run_fwd(op, inp, chunk)
    say(f"  rel err o={eo:.2e} ht={eh:.2e}")
    assert eo <= TOL[dt] and eh <= TOL[dt], (eo, eh)
