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

Prints one JSON line with the step throughput (tokens/s), a roofline entry
for the kernel that takes most of the step's time (its algorithmic bytes or
flops per launch over its average duration, timed with HIP events on its own
stream) and a CPU baseline (the fp64 oracle on a bounded sample).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
MFMA_FP32_PEAK_TFLOPS = 157.3
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
}


# workloads that time another op on an existing workload's inputs
CONFIG_OF = {"gdn_train_recompute_bf16_2k": "gdn_train_bf16_2k", "ssd_train_recompute_bf16_2k": "ssd_train_bf16_2k"}


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
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
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

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(e)


def kernel_model(name, c, esz=2, op="gdn_fwd + gdn_bwd"):
    """Algorithmic (bytes, flops) of one launch of a library kernel on workload c.

    Bytes: each tensor the kernel must read or write, counted once per
    launch (a tensor two workgroups both read counts once).  Flops: the dense
    GEMM products the kernel's step of the method needs (2*M*N*K each; the
    (I + A)^-1 solve and elementwise work excluded).  Per (token, head) terms
    scale with B*T*H, per-state terms (fp32 d_k x d_v) with B*H.
    """
    B, T, H, dk, dv, C = c["B"], c["T"], c["H"], c["dk"], c["dv"], c["chunk"]
    n_th, n_bh, st = B * T * H, B * H, dk * dv * 4
    e = esz
    per = {
        # whole forward: reads q, k, v, log_a, beta, h0; writes o, ht
        "k_fwd": ((2 * dk + dv) * e + 8 + dv * e, 2 * st,
                  2 * C * (3 * dk + 2 * dv) + 6 * dk * dv),
        # WY pass of the forward: reads q, k, v, log_a, beta; writes W, U'^T, g, P
        "k_wy": ((2 * dk + dv) * e + 8 + (dk + dv) * e + 4 + C * e, 0,
                 2 * C * dk + 2 * C * dk + 2 * C * dk + 2 * C * dv),
        # serial scan of the forward: reads q, k, W, U'^T, g, P, h0; writes o, ht
        "k_scan": (2 * dk * e + (dk + dv) * e + 4 + C * e + dv * e, 2 * st, 6 * dk * dv + 2 * C * dv),
        # WY pass of the backward recompute: reads q, k, v, log_a, beta; writes W, U'^T, g, Tinv, P
        "k_wy_bwd": ((2 * dk + dv) * e + 8 + (dk + dv) * e + 4 + C * e + C * e, 0,
                     2 * C * dk + 2 * C * dk + 2 * C * dk + 2 * C * dv),
        # scan of the backward recompute: reads k, W, U'^T, g, h0; writes U^T and the chunk-start states
        "k_scan_bwd": (2 * dk * e + dv * e + 4 + dv * e + dk * dv * e / C, st, 4 * dk * dv),
        # reads k, v, log_a, beta; writes W, U'^T, Ktil^T, g, Tinv
        "k_prep": ((dk + dv) * e + 8 + (2 * dk + dv) * e + 4 + C * e, 0,
                   2 * C * dk + 2 * C * dk + 2 * C * dv),
        # reads W, U'^T, Ktil^T, g, h0; writes U^T and the chunk-start states
        "k_state": ((2 * dk + dv) * e + 4 + dv * e + dk * dv * e / C, st, 4 * dk * dv),
        # reads q, k, do, g; writes dU_local
        "k_bwd_local": (2 * dk * e + 2 * dv * e + 4, 0, 2 * C * dk + 2 * C * dv),
        # reads q, k, do, g, W, P, dht; writes dU, the end-state gradients, dh0
        # (dU_local = P^T dO formed in the kernel)
        "k_dstate": (3 * dk * e + dv * e + C * e + 4 + dv * e + dk * dv * e / C, 2 * st,
                     6 * dk * dv + 2 * C * dv),
        # reads q, k, do, g, states, state gradients, U, dU; writes dq, dW, dK part, dg part
        "k_grad1": (2 * dk * e + dv * e + 4 + 2 * dk * dv * e / C + 2 * dv * e + 3 * dk * e + 4, 0,
                    2 * C * dk + 2 * C * dv + 2 * dk * dv + 2 * C * dk + 2 * dk * dv + 2 * dk * dv + 2 * C * dk),
        # reads k, v, beta, g, Tinv, dW, dU, dK part, dg part; writes dk, dv, dlog_a, dbeta
        "k_grad2": ((dk + dv) * e + 8 + C * e + dk * e + dv * e + dk * e + 4 + (dk + dv) * e + 8, 0,
                    2 * C * dk + 2 * C * dv + 2 * C * dk + 2 * C * dv + 4 * C * C + 2 * C * dk + 4 * C * dk),
    }
    if op == "gdn_fwd_train + gdn_bwd_saved":
        # the forward also keeps what the backward reads: the WY pass writes T
        # beside W, U'^T, g and P; the scan writes the chunk-start states and U^T
        b_th, b_bh, f_th = per["k_wy"]
        per["k_wy"] = (b_th + C * e, b_bh, f_th)
        b_th, b_bh, f_th = per["k_scan"]
        per["k_scan"] = (b_th + dk * dv * e / C + dv * e, b_bh, f_th)
    if op.startswith("ssd"):
        # the fused Mamba2 forward: reads q, k, v, log_a, h0; writes o, ht
        per["k_ssd_fwd"] = ((2 * dk + dv) * e + 4 + dv * e, 2 * st, 2 * C * (dk + dv) + 4 * dk * dv)
    if op.startswith("ssd_fwd_train"):
        # the training forward also writes the chunk-start states, g and P^T
        b_th, b_bh, f_th = per["k_ssd_fwd"]
        per["k_ssd_fwd"] = (b_th + dk * dv * e / C + 4 + C * e, b_bh, f_th)
    if op in ("ssd_fwd + ssd_bwd", "ssd_fwd_train + ssd_bwd_saved"):
        per.update({
            # reads v, log_a; writes g, V^T
            "k_ssd_prep": (dv * e + 4 + 4 + dv * e, 0, 0),
            # reads k, V^T, g, h0; writes the chunk-start states
            "k_scan_bwd": (dk * e + dv * e + 4 + dk * dv * e / C, st, 2 * dk * dv),
            # reads q, k, do, g, dU_local, dht; writes dU (= dv), the end-state gradients, dh0
            "k_dstate": (2 * dk * e + dv * e + 4 + dv * e + dv * e + dk * dv * e / C, 2 * st, 4 * dk * dv),
            # reads q, k, do, g, states, state gradients, V^T, dU; writes dq, dk, dv, dlog_a
            "k_grad1": (2 * dk * e + dv * e + 4 + 2 * dk * dv * e / C + 2 * dv * e + 2 * dk * e + dv * e + 4, 0,
                        6 * C * dk + 2 * C * dv + 4 * dk * dv),
        })
    if op == "ssd_fwd_train + ssd_bwd_saved":
        # reads q, k, do, g, the stored P^T, dht; writes dU (= dv), the end-state gradients, dh0
        per["k_dstate"] = (2 * dk * e + dv * e + 4 + C * e + dv * e + dk * dv * e / C, 2 * st,
                           4 * dk * dv + 2 * C * dv)
    if op == "kda_fwd":
        per.update({
            # reads q, k, v, per-dim log_a, beta; writes W, U'^T, Ktil^T, chunk decay, Q o e^G, P
            "k_kda_prep": ((2 * dk + dv) * e + dk * 4 + 4 + (2 * dk + dv) * e + dk * 4 / C + dk * e + C * e, 0,
                           2 * C * dk + 2 * C * dk + 2 * C * dk + 2 * C * dv),
            # reads W, U'^T, Ktil^T, chunk decay; writes U^T and the chunk-start states, ht
            "k_state": ((2 * dk + dv) * e + dk * 4 / C + dv * e + dk * dv * e / C, st, 4 * dk * dv),
            # reads Q o e^G, P, states, U; writes o
            "k_out": (dk * e + C * e + dk * dv * e / C + dv * e + dv * e, 0, 2 * C * dv + 2 * dk * dv),
        })
    if name not in per:
        return None
    b_th, b_bh, f_th = per[name]
    return b_th * n_th + b_bh * n_bh, f_th * n_th


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


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel factor), or
    None when there is none for this kernel or the sources have changed."""
    path = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("src_digest") != src_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else int(k["hbm_bytes_per_launch"])


def copy_probe(torch, dev, nbytes=1 << 30):
    """A plain device copy of known size, for scaling the byte counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def make_sets(L, synth, torch, wl, nsets):
    sets = []
    for s in range(nsets):
        inp = synth.config_inputs(wl, device="cuda", seed=s)
        sets.append(inp)
    return sets


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
    metric, op = WORKLOADS[wl]
    cfg = CONFIG_OF.get(wl, wl)
    c = dict(synth.CONFIGS[cfg])
    B, T, H, dk, dv, C = c["B"], c["T"], c["H"], c["dk"], c["dv"], c["chunk"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # input sets larger than the last-level cache need no rotation
    nsets = args.sets if B * T * H * (2 * dk + dv) * 2 < (1 << 30) else 1
    sets = make_sets(L, synth, torch, cfg, nsets)
    code = L.LRT_BF16
    opc = {"gdn_fwd + gdn_bwd": L.OP_GDN_BWD, "gdn_fwd_train + gdn_bwd_saved": L.OP_GDN_BWD, "gdn_fwd": L.OP_GDN_FWD, "ssd_fwd": L.OP_SSD_FWD,
           "ssd_fwd + ssd_bwd": L.OP_SSD_BWD, "ssd_fwd_train + ssd_bwd_saved": L.OP_SSD_BWD,
           "kda_fwd": L.OP_KDA_FWD}[op]
    ws_bytes = max(L.workspace_bytes(L.OP_GDN_FWD, B, T, H, dk, dv, C, code),
                   L.workspace_bytes(opc, B, T, H, dk, dv, C, code))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    grads = None
    if op.endswith(("_bwd", "_bwd_saved")):
        grads = (torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev),
                 torch.empty((B, T, H), dtype=torch.float32, device=dev),
                 torch.empty((B, T, H), dtype=torch.float32, device=dev),
                 torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev))
        if op.startswith("ssd"):
            grads = grads[:4] + grads[5:]

    def step(i):
        s = sets[i % len(sets)]
        if op == "ssd_fwd_train + ssd_bwd_saved":
            L.ssd_fwd_train(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), chunk=C, o=o, ht=ht, workspace=ws)
            L.ssd_bwd_saved(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), s["do"], ws, s.get("dht"), chunk=C,
                            out=grads)
            return
        if op.startswith("ssd"):
            L.ssd_fwd(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), chunk=C, o=o, ht=ht, workspace=ws)
        elif op == "gdn_fwd_train + gdn_bwd_saved":
            L.gdn_fwd_train(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                            workspace=ws)
            L.gdn_bwd_saved(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), s["do"], ws, s.get("dht"),
                            chunk=C, out=grads)
            return
        elif op == "kda_fwd":
            L.kda_fwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                      workspace=ws)
        else:
            L.gdn_fwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), chunk=C, o=o, ht=ht,
                      workspace=ws)
        if grads is not None and op.startswith("ssd"):
            L.ssd_bwd(s["q"], s["k"], s["v"], s["log_a"], s.get("h0"), s["do"], s.get("dht"), chunk=C, workspace=ws,
                      out=grads)
        elif grads is not None:
            L.gdn_bwd(s["q"], s["k"], s["v"], s["log_a"], s["beta"], s.get("h0"), s["do"], s.get("dht"),
                      chunk=C, workspace=ws, out=grads)

    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: throughput
    ev = hip.events(2)
    t0 = time.perf_counter()
    hip.lib.hipEventRecord(ctypes.c_void_p(ev[0]), ctypes.c_void_p(stream))
    for i in range(args.steps):
        step(i)
    hip.lib.hipEventRecord(ctypes.c_void_p(ev[1]), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = hip.elapsed_ms(ev[0], ev[1])
    hip.destroy(ev)
    ms_per_step = ms / args.steps
    tokens = B * T
    value = tokens * args.steps / (ms / 1e3)

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
    kernels = {n: {"launches": len(d), "avg_us": 1e3 * sum(d) / len(d), "total_us_per_step": 1e3 * sum(d) / args.steps}
               for n, d in dur.items()}
    dom = max(kernels, key=lambda n: kernels[n]["total_us_per_step"])
    model = kernel_model(dom, c, op=op)
    roof = None
    if model is not None:
        # every launch of a kernel in a step carries the same work
        per_launch_bytes, per_launch_flops = model
        avg_s = kernels[dom]["avg_us"] / 1e6
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        common = {"kernel": dom, "algorithmic_bytes": int(per_launch_bytes),
                  "algorithmic_flops": int(per_launch_flops), "avg_us": round(kernels[dom]["avg_us"], 2),
                  "traffic": counted_traffic(dom) if wl == WORKLOAD else None}
        if per_launch_flops / per_launch_bytes < ridge:
            ach = per_launch_bytes / avg_s / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), **common}
        else:
            ach = per_launch_flops / avg_s / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), **common}
    for n, k in kernels.items():
        m = kernel_model(n, c, op=op)
        if m is not None:
            k["gbs_algorithmic"] = m[0] / (k["avg_us"] / 1e6) / 1e9
            k["tflops_algorithmic"] = m[1] / (k["avg_us"] / 1e6) / 1e12

    # algorithmic step totals: GEMM flops of the method (forward, + backward)
    if op.startswith("ssd"):
        per_th = 2 * C * (dk + dv) + 4 * dk * dv
        if grads is not None:  # Mamba2 backward: 8 GEMM products, state recompute excluded
            per_th += 4 * C * dk + 4 * C * dv + 8 * dk * dv
    else:
        per_th = 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv
        if grads is not None:
            per_th += 12 * C * dk + 8 * C * dv + 12 * dk * dv + 4 * C * C
    step_tflops = per_th * B * T * H / (ms_per_step / 1e3) / 1e12

    cpu = None
    if not args.no_cpu_baseline and wl == WORKLOAD:
        cpu = cpu_baseline(sets[0], C, args.cpu_seconds)

    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded normal inputs; {nsets} rotating input set(s) resident in HBM)",
        "config": {"workload": wl, "B": B, "T": T, "H": H, "d_k": dk, "d_v": dv, "chunk": C, "op": op},
        "step_tflops": round(step_tflops, 2),
        "mfma_frac_of_bf16_peak": round(step_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "kernels": {n: {k: round(v, 2) if isinstance(v, float) else v for k, v in d.items()}
                    for n, d in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_probe:
        copy_probe(torch, dev)


def cpu_baseline(inp, C, target_s):
    """The fp64 oracle (forward + backward) on whole sequences of the first
    batch rows, adding rows until about target_s seconds of CPU work."""
    import oracle

    cpu = {k: (v.detach().cpu() if v is not None else None) for k, v in inp.items()}
    B, T, H = cpu["q"].shape[:3]
    cores = oracle.max_threads()
    per = max(1, min(B, -(-cores // H)))  # rows per call: enough (b, h) tasks for every core
    done_tokens, spent, rows = 0, 0.0, 0
    while rows < B and spent < target_s:
        sl = slice(rows, min(B, rows + per))
        a = {k: (v[sl].contiguous() if v is not None else None) for k, v in cpu.items()}
        t0 = time.perf_counter()
        oracle.fwd("gdn", a["q"], a["k"], a["v"], a["log_a"], a["beta"], a["h0"])
        oracle.bwd("gdn", a["q"], a["k"], a["v"], a["log_a"], a["beta"], a["h0"], a["do"], a.get("dht"))
        spent += time.perf_counter() - t0
        done_tokens += T * (sl.stop - sl.start)
        rows = sl.stop
    return {"value": round(done_tokens / spent, 1), "unit": "tokens/s", "cores": min(cores, per * H),
            "kind": "oracle",
            "sample": f"{rows} of {B} sequences x {T} tokens x {H} heads, fp64 forward + backward "
                      f"({spent:.1f} s)"}


if __name__ == "__main__":
    main()
