#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet training step on one MI355X.

One step = gdn_fwd_train + gdn_bwd_saved (the forward keeps the WY factors,
chunk-start states and new values the backward needs; the backward computes
all six gradients from them) over one batch of the pretraining-shaped
workload: B=16 sequences of T=2048 tokens, H=8 heads,
d_k = d_v = 128, chunk 64, bf16 tensors, fp32 gates and state (the shape of
the 2048-token bf16 runs on the AMD ROCm blog "Pretraining hybrid LLMs with
Primus", Table 4).  Inputs are synthetic (seeded), resident in HBM before the
timed region, and rotated over three independent sets so that no step reads
the previous step's inputs out of the 256 MB last-level cache.

Prints one JSON line:
  value / ms_per_step   step throughput (tokens/s) and its median, p10, p90;
  step                  the method's minimum HBM bytes and GEMM flops per step
                        (per (token, head): forward 1,032 B / 180,224 flop,
                        backward 1,808 B / 376,832 flop at d = 128, C = 64,
                        plus the fp32 states read and written) over the step
                        time, against 8 TB/s and 2,516.6 TFLOP/s; the
                        hardware-counter bytes of all the step's kernels when
                        counters of this build are committed;
  roofline              the kernel with the largest share of the step: the
                        method bytes of the pass it belongs to (forward or
                        backward) per launch over its average duration, timed
                        with HIP events on the launch stream;
  copy_gbs              a 1 GiB device copy timed in the same run;
  cpu_baseline          the fp64 oracle on a bounded sample, with the CPU model.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4,096 dense bf16 flop/clk/CU
WORKLOAD = "gdn_train_bf16_2k"  # the headline workload (default)
# the headline and other named workloads bench.py can time (context lines)
WORKLOADS = {
    "gdn_train_bf16_2k": ("GDN chunked fwd+bwd tokens/s and % bf16 MFMA peak, B=16 T=2048 H=8 d=128",
                          "gdn_fwd_train + gdn_bwd_saved"),
    # the same step through the stateless pair (the backward recomputes the forward)
    "gdn_train_recompute_bf16_2k": ("GDN chunked fwd+bwd (backward recomputes) tokens/s, B=16 T=2048 H=8 d=128",
                                    "gdn_fwd + gdn_bwd"),
    "gdn_bf16_2k": ("GDN chunked fwd tokens/s, B=16 T=2048 H=8 d=128", "gdn_fwd"),
    "ssd_bf16_2k": ("SSD (Mamba2 case) chunked fwd tokens/s, B=16 T=2048 H=8 d=128", "ssd_fwd"),
    "ssd_train_bf16_2k": ("SSD (Mamba2 case) chunked fwd+bwd tokens/s, B=16 T=2048 H=8 d=128",
                          "ssd_fwd_train + ssd_bwd_saved"),
    "ssd_train_recompute_bf16_2k": ("SSD (Mamba2 case) chunked fwd+bwd (backward recomputes) tokens/s, "
                                    "B=16 T=2048 H=8 d=128", "ssd_fwd + ssd_bwd"),
    "kda_bf16_1m": ("KDA chunked fwd tokens/s, B=1 T=2^20 H=16 d=128", "kda_fwd"),
    "kda_train_bf16_2k": ("KDA chunked fwd+bwd tokens/s, B=16 T=2048 H=8 d=128", "kda_fwd_train + kda_bwd_saved"),
    # the same step through the stateless pair (the backward recomputes the forward)
    "kda_train_recompute_bf16_2k": ("KDA chunked fwd+bwd (backward recomputes) tokens/s, B=16 T=2048 H=8 d=128",
                                    "kda_fwd + kda_bwd"),
    # the forwards on the raw projections, activations fused into the kernels
    # (the line also times the unfused pipeline: torch activations + the plain forward)
    "gdn_fused_bf16_2k": ("GDN chunked fwd, fused prologue (raw q/k/beta/gate in) tokens/s, B=16 T=2048 H=8 d=128",
                          "gdn_fwd_fused"),
    "kda_fused_bf16_1m": ("KDA chunked fwd, fused prologue (raw q/k/beta/gate in) tokens/s, B=1 T=2^20 H=16 d=128",
                          "kda_fwd_fused"),
    # the steps either side of the mixer: short conv on q/k/v and the gated output norm, fwd + bwd
    "conv_norm_bf16_2k": ("short conv (q, k, v) + gated RMSNorm fwd+bwd tokens/s, B=16 T=2048 H=8 d=128",
                          "short_conv fwd+bwd + gated_rmsnorm fwd+bwd"),
    # the same with the gate as its rank-16 factors (z = W_down x per token, W_up)
    "kda_fused_lowrank_bf16_1m": ("KDA chunked fwd, fused prologue with the rank-16 gate (raw q/k/beta, z, W_up in) "
                                  "tokens/s, B=1 T=2^20 H=16 d=128", "kda_fwd_fused_lowrank"),
}
# workloads that time another op on an existing workload's inputs
CONFIG_OF = {"gdn_train_recompute_bf16_2k": "gdn_train_bf16_2k", "ssd_train_recompute_bf16_2k": "ssd_train_bf16_2k",
             "kda_train_recompute_bf16_2k": "kda_train_bf16_2k",
             "gdn_fused_bf16_2k": "gdn_bf16_2k", "kda_fused_bf16_1m": "kda_bf16_1m",
             "kda_fused_lowrank_bf16_1m": "kda_bf16_1m"}

# the library kernels of each pass (the forward's and the backward's share of a step)
FWD_KERNELS = {"k_wy", "k_scan", "k_scan_local", "k_carry", "k_ssd_fwd", "k_kda_prep", "k_kda_prep_fast", "k_list_reset",
               "k_state_copy"}
# (k_kda_prep_bwd and k_kda_prep_fast_bwd are the backward's recompute of the KDA forward pass)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", default=WORKLOAD, choices=sorted(WORKLOADS))
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--sets", type=int, default=3, help="independent input sets rotated over the steps")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="finish with three 1 GiB device copies (scale of the byte counters)")
    return p.parse_args()


class Hip:
    """The few HIP runtime calls the timing needs (events), via ctypes."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            arr[i] = e.value
        return arr

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(e)


def method_model(op, c, has_h0, has_dht, esz=2):
    """The method's minimum HBM bytes and GEMM flops of each pass of `op` on
    workload c, per the per-(token, head) figures: every input read once and
    every output written once (q, k, v, gates, beta in; o out; for the
    backward also do in and dq, dk, dv and the gate/beta gradients out), plus
    the fp32 states (h0 / ht, dht / dh0) per (b, h); flops = the dense GEMM
    products of the chunkwise form (2*M*N*K each), no recompute.
    Returns {"fwd": (bytes, flops), "bwd": (bytes, flops)} (no "bwd" for a
    forward-only op)."""
    B, T, H, dk, dv, C = c["B"], c["T"], c["H"], c["dk"], c["dv"], c["chunk"]
    n_th, n_bh, st = B * T * H, B * H, dk * dv * 4
    e = esz
    ssd, kda = op.startswith("ssd"), op.startswith("kda")
    # the fused KDA forward reads the gate pre-activation in the call's dtype;
    # with the low-rank gate, 16 values per token shared by the H heads
    if kda and op.endswith("lowrank"):
        gate = 16 * e / H
    else:
        gate = (dk * e if op.endswith("fused") else 4 * dk) if kda else 4
    beta = 0 if ssd else 4
    fwd_b = (2 * dk + dv) * e + gate + beta + dv * e
    fwd_f = 2 * C * (dk + dv) + 4 * dk * dv if ssd else 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv
    out = {"fwd": (int(fwd_b * n_th) + (int(has_h0) + 1) * st * n_bh, fwd_f * n_th)}
    if "bwd" in op:
        # q, k, v, do, log a, beta in; dq, dk, dv, dlog_a, dbeta out (KDA: log a and dlog_a per key dim)
        g = 4 * dk if kda else 4
        bwd_b = (2 * dk + 2 * dv) * e + g + beta + (2 * dk + dv) * e + g + beta
        if ssd:
            bwd_f = 4 * C * dk + 4 * C * dv + 8 * dk * dv
        else:
            bwd_f = 12 * C * dk + 8 * C * dv + 12 * dk * dv + 4 * C * C
        out["bwd"] = (bwd_b * n_th + (int(has_h0) + int(has_dht) + 1) * st * n_bh, bwd_f * n_th)
    return out


def src_digest():
    """Digest of the HIP sources: hardware counters taken on another build
    do not describe this one."""
    import hashlib

    h = hashlib.sha256()
    d = os.path.join(ROOT, "linear_recurrent_token_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def counted_traffic(workload):
    """{kernel: HBM bytes per launch} from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE + WRITE_SIZE scaled by the
    copy-kernel factors), or None when there is none or the sources changed."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("src_digest") != src_digest():
        return None
    return {k: int(v["hbm_bytes_per_launch"]) for k, v in rec.get("kernels", {}).items()}


def copy_gbs(torch, hip, stream, dev, nbytes=1 << 30, reps=3):
    """A plain 1 GiB device copy (read + write), timed with HIP events: the
    achievable HBM bandwidth of this run.  Its buffers are freed after."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = hip.events(2)
    hip.record(ev[0], stream)
    for _ in range(reps):
        dst.copy_(src)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(ev[0], ev[1])
    hip.destroy(ev)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes * reps / (ms / 1e3) / 1e9


def copy_probe(torch, dev, nbytes=1 << 30):
    """Three plain device copies of known size, for scaling the byte counters
    of a rocprofv3 --pmc run."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def pct(xs, p):
    s = sorted(xs)
    i = min(len(s) - 1, max(0, int(round(p / 100.0 * (len(s) - 1)))))
    return s[i]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the mixer's hot path is measured on one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    import linear_recurrent_token_amd as L
    from linear_recurrent_token_amd import synth

    L.lib()
    wl = args.workload
    if wl == "conv_norm_bf16_2k":
        return main_conv_norm(args, wl)
    metric, op = WORKLOADS[wl]
    cfg = CONFIG_OF.get(wl, wl)
    c = dict(synth.CONFIGS[cfg])
    B, T, H, dk, dv, C = c["B"], c["T"], c["H"], c["dk"], c["dv"], c["chunk"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    copy = copy_gbs(torch, hip, stream, dev)
    # input sets larger than the last-level cache need no rotation
    nsets = args.sets if B * T * H * (2 * dk + dv) * 2 < (1 << 30) else 1
    fused = op.endswith("_fused") or op.endswith("_lowrank")
    if fused:
        sets = [synth.raw_inputs(cfg, device="cuda", seed=s, lowrank_factors_too=op.endswith("_lowrank"))
                for s in range(nsets)]
    else:
        sets = [synth.config_inputs(cfg, device="cuda", seed=s) for s in range(nsets)]
    code = L.LRT_BF16
    opc = {"gdn_fwd + gdn_bwd": L.OP_GDN_BWD, "gdn_fwd_train + gdn_bwd_saved": L.OP_GDN_BWD, "gdn_fwd": L.OP_GDN_FWD,
           "ssd_fwd": L.OP_SSD_FWD, "ssd_fwd + ssd_bwd": L.OP_SSD_BWD, "ssd_fwd_train + ssd_bwd_saved": L.OP_SSD_BWD,
           "kda_fwd": L.OP_KDA_FWD, "gdn_fwd_fused": L.OP_GDN_FWD, "kda_fwd_fused": L.OP_KDA_FWD,
           "kda_fwd_fused_lowrank": L.OP_KDA_FWD,
           "kda_fwd + kda_bwd": L.OP_KDA_BWD, "kda_fwd_train + kda_bwd_saved": L.OP_KDA_BWD}[op]
    ws_bytes = max(L.workspace_bytes(L.OP_KDA_FWD if op.startswith("kda") else L.OP_GDN_FWD, B, T, H, dk, dv, C,
                                     code), L.workspace_bytes(opc, B, T, H, dk, dv, C, code))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    grads = None
    if "bwd" in op:
        grads = (torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, T, H, dk) if op.startswith("kda") else (B, T, H), dtype=torch.float32, device=dev),
                 torch.empty((B, T, H), dtype=torch.float32, device=dev),
                 torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev))
        if op.startswith("ssd"):
            grads = grads[:4] + grads[5:]

    def activate(s):
        """The unfused pipeline's activation passes (torch), for the comparison line."""
        def l2(x):
            x = x.float()
            return (x / torch.sqrt((x * x).sum(-1, keepdim=True) + 1e-6)).to(x_dtype)
        x_dtype = s["q_raw"].dtype
        if "z" in s:  # the low-rank gate: W_up z first (a torch GEMM)
            B_, T_, H_, dk_ = s["q_raw"].shape
            pre = (s["z"].view(B_ * T_, -1) @ s["w_up"].t()).view(B_, T_, H_, dk_)
        else:
            pre = s["gate_raw"]
        return (l2(s["q_raw"]), l2(s["k_raw"]), -torch.nn.functional.softplus(pre.float()),
                torch.sigmoid(s["beta_raw"]))

    def step_unfused(i):
        s = sets[i % len(sets)]
        q, k, la, beta = activate(s)
        f = L.kda_fwd if op.startswith("kda") else L.gdn_fwd
        f(q, k, s["v"], la, beta, s.get("h0"), chunk=C, o=o, ht=ht, workspace=ws)

    def step(i):
        s = sets[i % len(sets)]
        if op == "kda_fwd_fused_lowrank":
            L.kda_fwd_fused_lowrank(s["q_raw"], s["k_raw"], s["v"], s["z"], s["w_up"], s["beta_raw"], s.get("h0"),
                                    chunk=C, o=o, ht=ht, workspace=ws)
            return
        if fused:
            f = L.kda_fwd_fused if op == "kda_fwd_fused" else L.gdn_fwd_fused
            f(s["q_raw"], s["k_raw"], s["v"], s["gate_raw"], s["beta_raw"], s.get("h0"), chunk=C, o=o, ht=ht,
              workspace=ws)
            return
        if op == "ssd_fwd_train + ssd_bwd_saved":
            L.ssd_fwd_train(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), chunk=C, o=o, ht=ht, workspace=ws)
            L.ssd_bwd_saved(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), s["do"], ws, s.get("dht"), chunk=C,
                            out=grads)
            return
        if op == "kda_fwd_train + kda_bwd_saved":
            L.kda_fwd_train(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                            workspace=ws)
            L.kda_bwd_saved(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), s["do"], ws, s.get("dht"),
                            chunk=C, out=grads)
            return
        if op == "gdn_fwd_train + gdn_bwd_saved":
            L.gdn_fwd_train(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                            workspace=ws)
            L.gdn_bwd_saved(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), s["do"], ws, s.get("dht"),
                            chunk=C, out=grads)
            return
        if op.startswith("ssd"):
            L.ssd_fwd(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), chunk=C, o=o, ht=ht, workspace=ws)
        elif op.startswith("kda"):
            L.kda_fwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                      workspace=ws)
        else:
            L.gdn_fwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                      workspace=ws)
        if grads is not None and op.startswith("ssd"):
            L.ssd_bwd(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), s["do"], s.get("dht"), chunk=C, workspace=ws,
                      out=grads)
        elif grads is not None and op.startswith("kda"):
            L.kda_bwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), s["do"], s.get("dht"),
                      chunk=C, workspace=ws, out=grads)
        elif grads is not None:
            L.gdn_bwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), s["do"], s.get("dht"),
                      chunk=C, workspace=ws, out=grads)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: throughput, one event per step boundary
    ev = hip.events(args.steps + 1)
    t0 = time.perf_counter()
    hip.record(ev[0], stream)
    for i in range(args.steps):
        step(i)
        hip.record(ev[i + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [hip.elapsed_ms(ev[i], ev[i + 1]) for i in range(args.steps)]
    ms = hip.elapsed_ms(ev[0], ev[args.steps])
    hip.destroy(ev)
    ms_per_step = ms / args.steps
    value = B * T * args.steps / (ms / 1e3)

    # timed region again, every library kernel bracketed by HIP events
    per_step_kernels = 16
    nk = per_step_kernels * args.steps
    kev = hip.events(2 * nk)
    kinds = (ctypes.c_int * nk)()
    L.lib().lrt_profile_attach(ctypes.cast(kev, ctypes.c_void_p), ctypes.cast(kinds, ctypes.c_void_p), nk)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    n_rec = L.lib().lrt_profile_count()
    L.lib().lrt_profile_attach(None, None, 0)
    dur = {}
    for i in range(n_rec):
        name = L.lib().lrt_kernel_name(kinds[i]).decode()
        dur.setdefault(name, []).append(hip.elapsed_ms(kev[2 * i], kev[2 * i + 1]))
    hip.destroy(kev)
    kernels = {n: {"launches": len(d), "avg_us": 1e3 * sum(d) / len(d),
                   "total_us_per_step": 1e3 * sum(d) / args.steps} for n, d in dur.items()}

    has_h0 = sets[0].get("h0") is not None
    has_dht = sets[0].get("dht") is not None
    model = method_model(op, c, has_h0, has_dht)
    step_bytes = sum(b for b, _ in model.values())
    step_flops = sum(f for _, f in model.values())
    step_s = ms_per_step / 1e3
    traffic = counted_traffic(wl)
    traffic_total = None
    if traffic is not None and all(n in traffic for n in kernels):
        traffic_total = int(sum(traffic[n] * k["launches"] / args.steps for n, k in kernels.items()))
    for n, k in kernels.items():
        k["share_of_step"] = k["total_us_per_step"] / 1e3 / ms_per_step
        if traffic is not None and n in traffic:
            k["counted_bytes_per_launch"] = traffic[n]
            k["counted_gbs"] = traffic[n] / (k["avg_us"] / 1e6) / 1e9

    dom = max(kernels, key=lambda n: kernels[n]["total_us_per_step"])
    pas = "fwd" if dom in FWD_KERNELS or "bwd" not in model else "bwd"
    mb, mf = model[pas]
    avg_s = kernels[dom]["avg_us"] / 1e6
    launches = kernels[dom]["launches"] / args.steps  # launches per step: the pass's units split among them
    mb_launch, mf_launch = mb / launches, mf / launches
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    common = {"kernel": dom, "pass": pas, "method_bytes_per_launch": int(mb_launch),
              "method_flops_per_launch": int(mf_launch), "avg_us": round(kernels[dom]["avg_us"], 2),
              "traffic": traffic.get(dom) if traffic is not None else None}
    if mf_launch / mb_launch < ridge:
        ach = mb_launch / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), **common}
    else:
        ach = mf_launch / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), **common}

    unfused = None
    if fused:
        # the same step through the unfused pipeline (activation passes + plain forward), same events
        for i in range(2):
            step_unfused(i)
        torch.cuda.synchronize()
        ev = hip.events(2)
        hip.record(ev[0], stream)
        for i in range(args.steps):
            step_unfused(i)
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        ums = hip.elapsed_ms(ev[0], ev[1]) / args.steps
        hip.destroy(ev)
        unfused = {"ms_per_step": round(ums, 4), "fused_speedup": round(ums / ms_per_step, 3),
                   "what": ("torch " + ("gate = W_up z (GEMM), " if op.endswith("_lowrank") else "")
                            + "l2norm(q), l2norm(k), -softplus(gate), sigmoid(beta) then the plain forward")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu_inp = sets[0]
        if fused:
            q, k, la, beta = activate(sets[0])
            cpu_inp = {"q": q, "k": k, "v": sets[0]["v"], "log_a": la, "beta": beta, "h0": sets[0].get("h0")}
        cpu = cpu_baseline(op, cpu_inp, C, args.cpu_seconds)

    step_rec = {
        "method_bytes": int(step_bytes),
        "method_flops": int(step_flops),
        "hbm_gbs": round(step_bytes / step_s / 1e9, 1),
        "hbm_frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_frac_of_copy": round(step_bytes / step_s / 1e9 / copy, 4),
        "tflops": round(step_flops / step_s / 1e12, 2),
        "mfma_frac": round(step_flops / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "traffic_total": traffic_total,
        "kernel_us_sum": round(sum(k["total_us_per_step"] for k in kernels.values()), 2),
    }
    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_p10": round(pct(per, 10), 4),
        "ms_per_step_p50": round(pct(per, 50), 4),
        "ms_per_step_p90": round(pct(per, 90), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded normal inputs; {nsets} rotating input set(s) resident in HBM)",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "d_k": dk, "d_v": dv, "chunk": C, "op": op},
        "step": step_rec,
        "mfma_frac_of_bf16_peak": step_rec["mfma_frac"],
        "copy_gbs": round(copy, 1),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "kernels": {n: {k: round(v, 4) if isinstance(v, float) else v for k, v in d.items()}
                    for n, d in kernels.items()},
        "cpu_baseline": cpu,
    }
    if unfused is not None:
        line["unfused_pipeline"] = unfused
    print(json.dumps(line), flush=True)
    if args.copy_probe:
        copy_probe(torch, dev)


def main_conv_norm(args, wl):
    """The steps either side of the mixer in one training step of the
    2048-token workload: short_conv fwd + bwd over q, k and v as the 3 x 1024
    columns of one [16, 2048, 3072] tensor (W = 4), and gated_rmsnorm fwd + bwd
    over the mixer output [16, 2048, 8, 128].  Each kernel is an exact stream,
    so its method bytes are its own reads and writes.  Also timed: the same
    step through torch (conv1d + silu, rms_norm * silu, autograd)."""
    import torch
    import torch.nn.functional as F

    import linear_recurrent_token_amd as L

    L.lib()
    metric, op = WORKLOADS[wl]
    B, T, H, d, W = 16, 2048, 8, 128, 4
    D = 3 * H * d
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    copy = copy_gbs(torch, hip, stream, dev)
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((B, T, D), generator=g, device=dev).to(torch.bfloat16)
    dy = torch.randn((B, T, D), generator=g, device=dev).to(torch.bfloat16)
    wc = 0.5 * torch.randn((D, W), generator=g, device=dev)
    o = torch.randn((B, T, H, d), generator=g, device=dev).to(torch.bfloat16)
    z = torch.randn((B, T, H, d), generator=g, device=dev).to(torch.bfloat16)
    dyn = torch.randn((B, T, H, d), generator=g, device=dev).to(torch.bfloat16)
    wn = 1.0 + 0.1 * torch.randn((d,), generator=g, device=dev)
    wsc = torch.empty(L.lib().short_conv_bwd_workspace_bytes(B * T, D, W), dtype=torch.uint8, device=dev)
    wsn = torch.empty(L.lib().gated_rmsnorm_bwd_workspace_bytes(B * T * H, d), dtype=torch.uint8, device=dev)

    def step(i):
        L.short_conv(x, wc)
        L.short_conv_bwd(x, wc, dy, workspace=wsc)
        L.gated_rmsnorm(o, z, wn)
        L.gated_rmsnorm_bwd(o, z, wn, dyn, workspace=wsn)

    def step_torch(i):
        xs = x.detach().requires_grad_(True)
        ws = wc.detach().requires_grad_(True)
        pre = F.conv1d(xs.transpose(1, 2), ws.to(x.dtype).view(D, 1, W), padding=W - 1, groups=D)[..., :T]
        yc = F.silu(pre).transpose(1, 2)
        os_, zs, wns = o.detach().requires_grad_(True), z.detach().requires_grad_(True), wn.detach().requires_grad_(True)
        yn = F.rms_norm(os_, (d,), weight=wns.to(o.dtype), eps=1e-6) * F.silu(zs)
        torch.autograd.backward([yc, yn], [dy, dyn])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = hip.events(args.steps + 1)
    t0 = time.perf_counter()
    hip.record(ev[0], stream)
    for i in range(args.steps):
        step(i)
        hip.record(ev[i + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [hip.elapsed_ms(ev[i], ev[i + 1]) for i in range(args.steps)]
    ms = hip.elapsed_ms(ev[0], ev[args.steps])
    hip.destroy(ev)
    ms_per_step = ms / args.steps
    value = B * T * args.steps / (ms / 1e3)

    nk = 8 * args.steps
    kev = hip.events(2 * nk)
    kinds = (ctypes.c_int * nk)()
    L.lib().lrt_profile_attach(ctypes.cast(kev, ctypes.c_void_p), ctypes.cast(kinds, ctypes.c_void_p), nk)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    n_rec = L.lib().lrt_profile_count()
    L.lib().lrt_profile_attach(None, None, 0)
    dur = {}
    for i in range(n_rec):
        dur.setdefault(L.lib().lrt_kernel_name(kinds[i]).decode(), []).append(hip.elapsed_ms(kev[2 * i], kev[2 * i + 1]))
    hip.destroy(kev)
    kernels = {n: {"launches": len(v), "avg_us": 1e3 * sum(v) / len(v), "total_us_per_step": 1e3 * sum(v) / args.steps}
               for n, v in dur.items()}
    # each kernel's method bytes per launch: its reads and writes of the token tensors (bf16)
    xb, nb_ = B * T * D * 2, B * T * H * d * 2
    own = {"k_conv_fwd": 2 * xb, "k_conv_bwd": 3 * xb, "k_gnorm_fwd": 3 * nb_, "k_gnorm_bwd": 5 * nb_,
           "k_rows_reduce(conv dw)": 0, "k_rows_reduce(norm dw)": 0}
    step_bytes = sum(own.get(n, 0) * k["launches"] / args.steps for n, k in kernels.items())
    for n, k in kernels.items():
        k["share_of_step"] = k["total_us_per_step"] / 1e3 / ms_per_step
        if own.get(n):
            k["method_gbs"] = own[n] / (k["avg_us"] / 1e6) / 1e9
    dom = max(kernels, key=lambda n: kernels[n]["total_us_per_step"])
    ach = own[dom] / (kernels[dom]["avg_us"] / 1e6) / 1e9
    traffic = counted_traffic(wl)
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic.get(dom) if traffic is not None else None,
            "kernel": dom, "method_bytes_per_launch": int(own[dom]), "avg_us": round(kernels[dom]["avg_us"], 2)}

    for i in range(2):
        step_torch(i)
    torch.cuda.synchronize()
    ev = hip.events(2)
    hip.record(ev[0], stream)
    for i in range(args.steps):
        step_torch(i)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    tms = hip.elapsed_ms(ev[0], ev[1]) / args.steps
    hip.destroy(ev)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle.conv_norm as cn
        t1, rows = time.perf_counter(), 0
        while rows < B and time.perf_counter() - t1 < args.cpu_seconds:
            sl = slice(rows, rows + 1)
            cn.short_conv(x[sl], wc)
            cn.short_conv_bwd(x[sl], wc, dy[sl])
            cn.gated_rmsnorm(o[sl], z[sl], wn)
            cn.gated_rmsnorm_bwd(o[sl], z[sl], wn, dyn[sl])
            rows += 1
        spent = time.perf_counter() - t1
        cpu = {"value": round(rows * T / spent, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"{rows} of {B} sequences x {T} tokens, all channels, fp64 numpy ({spent:.1f} s)"}

    line = {
        "metric": metric, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "ms_per_step_p10": round(pct(per, 10), 4),
        "ms_per_step_p50": round(pct(per, 50), 4), "ms_per_step_p90": round(pct(per, 90), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal inputs resident in HBM)",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "d": d, "conv_channels": D, "conv_width": W, "op": op},
        "step": {"method_bytes": int(step_bytes), "hbm_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
                 "hbm_frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "hbm_frac_of_copy": round(step_bytes / (ms_per_step / 1e3) / 1e9 / copy, 4)},
        "copy_gbs": round(copy, 1), "wall_s_timed": round(wall, 4), "roofline": roof,
        "kernels": {n: {k: round(v, 4) if isinstance(v, float) else v for k, v in dd.items()}
                    for n, dd in kernels.items()},
        "unfused_pipeline": {"ms_per_step": round(tms, 4), "fused_speedup": round(tms / ms_per_step, 3),
                             "what": "torch conv1d (groups = channels) + silu and rms_norm * silu, with autograd"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_probe:
        copy_probe(torch, dev)


def cpu_baseline(op, inp, C, target_s):
    """The fp64 oracle on a bounded sample of the workload: whole sequences of
    the first batch rows (forward, plus the backward for a training step),
    adding rows until about target_s seconds of CPU work; for a single long
    sequence, a prefix of it doubled in length until the target is reached."""
    import oracle

    variant = "ssd" if op.startswith("ssd") else "kda" if op.startswith("kda") else "gdn"
    train = "bwd" in op
    cpu = {k: (v.detach().cpu() if v is not None and k != "qidx" else None) for k, v in inp.items()}
    B, T, H = cpu["q"].shape[:3]
    cores = oracle.max_threads()

    def run(a):
        t0 = time.perf_counter()
        oracle.fwd(variant, a["q"], a["k"], a["v"], a["log_a"], a.get("beta"), a.get("h0"))
        if train:
            oracle.bwd(variant, a["q"], a["k"], a["v"], a["log_a"], a.get("beta"), a.get("h0"), a["do"], a.get("dht"))
        return time.perf_counter() - t0

    what = "forward + backward" if train else "forward"
    if B == 1:
        n, spent, done = 1024, 0.0, 0
        while True:
            a = {k: (v[:, :n].contiguous() if v is not None and v.dim() >= 3 and v.shape[1] == T else v)
                 for k, v in cpu.items()}
            spent = run(a)
            done = n
            if spent >= target_s / 2 or n >= T:
                break
            n = min(T, n * 2)
        sample = f"first {done} of {T} tokens x {H} heads, fp64 {what} ({spent:.1f} s)"
        tok = done
        used = min(cores, H)
    else:
        per = max(1, min(B, -(-cores // H)))  # rows per call: enough (b, h) tasks for every core
        tok, spent, rows = 0, 0.0, 0
        while rows < B and spent < target_s:
            sl = slice(rows, min(B, rows + per))
            a = {k: (v[sl].contiguous() if v is not None else None) for k, v in cpu.items()}
            spent += run(a)
            tok += T * (sl.stop - sl.start)
            rows = sl.stop
        sample = f"{rows} of {B} sequences x {T} tokens x {H} heads, fp64 {what} ({spent:.1f} s)"
        used = min(cores, per * H)
    return {"value": round(tok / spent, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(), "sample": sample}


if __name__ == "__main__":
    main()
