"""Seeded synthetic inputs for the gated delta-rule mixers.

This module holds no arithmetic of the mixers themselves: it only draws the
tensors that both the GPU library and the CPU oracle are fed.  The shapes and
distributions follow the workloads on the AMD ROCm blog "Pretraining hybrid
LLMs with Primus" (Table 4: sequence length 2048, bf16) and the 1M-token
long-context guide for the 7-MLA/21-GDN hybrid (16 heads, 1,048,576 tokens);
FineWeb-Edu text and trained projections are replaced by random tensors of
those shapes.

Every tensor gets its own ``torch.Generator`` seeded from (seed, slot), so a
tensor's values do not depend on which other tensors were drawn.  Values are
drawn in fp32 on ``device``, derived in fp32 (L2 normalisation, sigmoid,
softplus) and only then cast to the storage dtype.
"""
from __future__ import annotations

import torch

# slot numbers: fixed, so that adding a tensor never changes another's values
_SLOTS = {"q": 1, "k": 2, "v": 3, "beta": 4, "gate": 5, "h0": 6, "do": 7, "dht": 8,
          "x": 9, "w_down": 10, "w_up": 11}

# Named workloads.  gate: shift s of log a = -softplus(N(0,1) + s); h0_std 0 = no state.
CONFIGS = {
    # gated delta rule forward, fp32, tiny
    "gdn_fp32_tiny": dict(op="gdn_fwd", B=1, T=64, H=2, dk=16, dv=16, chunk=16,
                          dtype=torch.float32, gate_shift=0.0, h0_std=0.0),
    # Mamba2 / SSD forward at the pretraining shape
    "ssd_bf16_2k": dict(op="ssd_fwd", B=16, T=2048, H=8, dk=128, dv=128, chunk=64,
                        dtype=torch.bfloat16, gate_shift=0.0, h0_std=0.0),
    # Gated DeltaNet forward at the pretraining shape
    "gdn_bf16_2k": dict(op="gdn_fwd", B=16, T=2048, H=8, dk=128, dv=128, chunk=64,
                        dtype=torch.bfloat16, gate_shift=2.0, h0_std=0.1),
    # Gated DeltaNet training step (forward + backward) at the pretraining shape
    "gdn_train_bf16_2k": dict(op="gdn_fwd_bwd", B=16, T=2048, H=8, dk=128, dv=128, chunk=64,
                              dtype=torch.bfloat16, gate_shift=2.0, h0_std=0.1),
    # Mamba2 / SSD training step (forward + backward) at the pretraining shape,
    # with the Mamba2 forward's distributions
    "ssd_train_bf16_2k": dict(op="ssd_fwd_bwd", B=16, T=2048, H=8, dk=128, dv=128, chunk=64,
                              dtype=torch.bfloat16, gate_shift=0.0, h0_std=0.0),
    # Kimi Delta Attention training step (forward + backward) at the 2048-token
    # pretraining shape, the rank-16 low-rank per-dimension gate
    "kda_train_bf16_2k": dict(op="kda_fwd_bwd", B=16, T=2048, H=8, dk=128, dv=128, chunk=64,
                              dtype=torch.bfloat16, gate="lowrank", rank=16, h0_std=0.1),
    # Kimi Delta Attention forward over one 1M-token sequence, 16 heads
    "kda_bf16_1m": dict(op="kda_fwd", B=1, T=1 << 20, H=16, dk=128, dv=128, chunk=64,
                        dtype=torch.bfloat16, gate="lowrank", rank=16, h0_std=0.0),
}


def _gen(seed: int, slot: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + _SLOTS[slot])
    return g


def randn(shape, seed, slot, device="cpu", std=1.0, mean=0.0):
    g = _gen(seed, slot, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x


def _unit_rows(x):
    # L2 normalisation over the last dim, in fp32, no epsilon (N(0,1) rows are never zero)
    return x / x.norm(dim=-1, keepdim=True)


def orthonormal_keys(B, T, H, dk, seed, device="cpu"):
    """Keys k_t, t < T <= dk, that are rows of one random orthogonal dk x dk
    matrix per (b, h) (QR of a Gaussian matrix in fp64), as [B, T, H, dk]
    fp32, and query indices j(t) drawn uniformly from [0, t] (int64 [B, T, H])."""
    if T > dk:
        raise ValueError("orthonormal keys need T <= d_k")
    g = torch.Generator().manual_seed(int(seed) * 1000003 + _SLOTS["k"])
    z = torch.randn((B, H, dk, dk), generator=g, dtype=torch.float64)
    qmat, r = torch.linalg.qr(z)
    qmat = qmat * torch.sign(torch.diagonal(r, dim1=-2, dim2=-1)).unsqueeze(-2)
    keys = qmat.transpose(-1, -2)[:, :, :T, :].permute(0, 2, 1, 3).contiguous()  # rows -> [B, T, H, dk]
    gq = torch.Generator().manual_seed(int(seed) * 1000003 + _SLOTS["q"])
    u = torch.rand((B, T, H), generator=gq, dtype=torch.float64)
    idx = torch.floor(u * (torch.arange(T, dtype=torch.float64).view(1, T, 1) + 1)).long()
    return keys.to(torch.float32).to(device), idx.to(device)


def make_inputs(op, B, T, H, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu",
                gate_shift=0.0, h0_std=0.0, gate="scalar", rank=16, gate_width=None,
                with_do=False, dht_std=0.0, chunk=None, beta_shift=0.0, beta_kind="sigmoid",
                keys="normal"):
    """Draw inputs for ``op`` in {'gdn_fwd', 'gdn_fwd_bwd', 'ssd_fwd', 'ssd_fwd_bwd', 'kda_fwd'}.

    Returns a dict with q, k, v [B,T,H,d] in ``dtype``; log_a fp32 [B,T,H]
    ([B,T,H,dk] for KDA); beta fp32 [B,T,H] (absent for SSD); h0 fp32
    [B,H,dk,dv] or None; do (``dtype``) and dht (fp32 or None) when asked.

    gate:
      'scalar'  log a = -softplus(N(0,1) + gate_shift), one per (b,t,h)
      'perdim'  the same, drawn i.i.d. per key dimension (KDA only)
      'uniform' KDA gate equal over the key dimensions (one scalar broadcast)
      'lowrank' log a = -softplus(W_up (W_down x)), x ~ N(0,1) of width
                ``gate_width`` (default H*dk), W ~ 0.02 N(0,1), rank ``rank``;
                computed in fp32 on ``device`` in blocks of tokens.
      'zero'    log a = 0 (no decay)
    beta_kind: 'sigmoid' (b = sigmoid(N(0,1) + beta_shift)) or 'one' (b = 1).
    keys: 'normal' (q, k ~ N(0,1), L2-normalised) or 'orthonormal' (k_t rows
          of a random orthogonal matrix per (b, h), T <= d_k, and q_t = k_j(t)
          with j(t) uniform in [0, t]; the indices are returned as 'qidx').
    """
    kda = op.startswith("kda")
    out = {}
    if keys == "orthonormal":
        kk, idx = orthonormal_keys(B, T, H, dk, seed, device)
        out["k"] = kk.to(dtype)
        out["q"] = torch.gather(kk, 1, idx[..., None].expand(B, T, H, dk)).to(dtype)
        out["qidx"] = idx
    else:
        out["q"] = _unit_rows(randn((B, T, H, dk), seed, "q", device)).to(dtype)
        out["k"] = _unit_rows(randn((B, T, H, dk), seed, "k", device)).to(dtype)
    out["v"] = randn((B, T, H, dv), seed, "v", device).to(dtype)
    if not op.startswith("ssd"):
        if beta_kind == "one":
            out["beta"] = torch.ones((B, T, H), dtype=torch.float32, device=device)
        else:
            out["beta"] = torch.sigmoid(randn((B, T, H), seed, "beta", device) + beta_shift)
    if gate == "zero":
        out["log_a"] = torch.zeros((B, T, H, dk) if kda else (B, T, H), dtype=torch.float32, device=device)
    elif kda and gate == "lowrank":
        out["log_a"] = lowrank_gate(B, T, H, dk, seed, device, rank=rank, width=gate_width)
    elif kda and gate == "perdim":
        out["log_a"] = -torch.nn.functional.softplus(randn((B, T, H, dk), seed, "gate", device) + gate_shift)
    else:
        la = -torch.nn.functional.softplus(randn((B, T, H), seed, "gate", device) + gate_shift)
        out["log_a"] = la[..., None].expand(B, T, H, dk).contiguous() if kda else la
    out["h0"] = randn((B, H, dk, dv), seed, "h0", device, std=h0_std) if h0_std > 0 else None
    if with_do or op.endswith("bwd"):
        out["do"] = randn((B, T, H, dv), seed, "do", device).to(dtype)
        out["dht"] = randn((B, H, dk, dv), seed, "dht", device, std=dht_std) if dht_std > 0 else None
    return out


def lowrank_gate(B, T, H, dk, seed, device, rank=16, width=None, block=1 << 16, preact=False,
                 out_dtype=torch.float32):
    """log a = -softplus(W_up (W_down x)) in fp32, [B,T,H,dk]; x drawn per token block.
    preact=True returns the pre-activation W_up (W_down x) itself (in out_dtype)."""
    D = H * dk if width is None else int(width)
    w_down = randn((rank, D), seed, "w_down", device, std=0.02)
    w_up = randn((H * dk, rank), seed, "w_up", device, std=0.02)
    out = torch.empty((B, T, H, dk), dtype=out_dtype, device=device)
    g = _gen(seed, "x", device)
    for b in range(B):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            x = torch.randn((t1 - t0, D), generator=g, device=device, dtype=torch.float32)
            z = (x @ w_down.t()) @ w_up.t()
            out[b, t0:t1] = (z if preact else -torch.nn.functional.softplus(z)).view(t1 - t0, H, dk).to(out_dtype)
    return out


def lowrank_factors(B, T, H, dk, seed, device, rank=16, width=None, block=1 << 16, out_dtype=torch.bfloat16):
    """The low-rank gate's factors, drawn as lowrank_gate draws them: z = W_down x
    [B, T, rank] (each token's bottleneck activations) and W_up [H*dk, rank],
    both in out_dtype; the gate pre-activation is W_up z."""
    D = H * dk if width is None else int(width)
    w_down = randn((rank, D), seed, "w_down", device, std=0.02)
    w_up = randn((H * dk, rank), seed, "w_up", device, std=0.02)
    z = torch.empty((B, T, rank), dtype=out_dtype, device=device)
    g = _gen(seed, "x", device)
    for b in range(B):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            x = torch.randn((t1 - t0, D), generator=g, device=device, dtype=torch.float32)
            z[b, t0:t1] = (x @ w_down.t()).to(out_dtype)
    return z, w_up.to(out_dtype)


def raw_inputs(name, device="cpu", seed=0, lowrank_factors_too=False):
    """The raw projections of a named workload, for the fused-prologue entry
    points: q_raw, k_raw ~ N(0,1) (not normalised), v, beta_raw ~ N(0,1)
    (the beta logits), gate_raw = the gate pre-activation (fp32 N(0,1) +
    gate_shift for a scalar gate; the rank-16 projection W_up (W_down x) in
    the workload's dtype for KDA -- or, with lowrank_factors_too, its factors
    z = W_down x and W_up instead), h0."""
    c = dict(CONFIGS[name])
    B, T, H, dk, dv, dtype = c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"]
    out = {"q_raw": randn((B, T, H, dk), seed, "q", device).to(dtype),
           "k_raw": randn((B, T, H, dk), seed, "k", device).to(dtype),
           "v": randn((B, T, H, dv), seed, "v", device).to(dtype),
           "beta_raw": randn((B, T, H), seed, "beta", device)}
    if c.get("gate") == "lowrank" and lowrank_factors_too:
        out["z"], out["w_up"] = lowrank_factors(B, T, H, dk, seed, device, rank=c.get("rank", 16), out_dtype=dtype)
    elif c.get("gate") == "lowrank":
        out["gate_raw"] = lowrank_gate(B, T, H, dk, seed, device, rank=c.get("rank", 16), preact=True,
                                       out_dtype=dtype)
    else:
        out["gate_raw"] = randn((B, T, H), seed, "gate", device, mean=c.get("gate_shift", 0.0))
    h0s = c.get("h0_std", 0.0)
    out["h0"] = randn((B, H, dk, dv), seed, "h0", device, std=h0s) if h0s > 0 else None
    return out


def config_inputs(name, device="cpu", seed=0, **over):
    """Inputs of a named workload (see CONFIGS); keyword overrides allowed."""
    c = dict(CONFIGS[name])
    c.update(over)
    op = c.pop("op")
    c.pop("dtype", None)
    dtype = over.get("dtype", CONFIGS[name]["dtype"])
    c.pop("chunk", None)
    return make_inputs(op, dtype=dtype, seed=seed, device=device, **c)
