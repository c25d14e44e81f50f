"""fp64 CPU oracle for the gated delta-rule token mixers (GDN, SSD, KDA).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline may import this package; the product library and its Python binding
never do.  It shares no code with the GPU path.

The arithmetic lives in ``oracle.c`` (plain sequential recurrence in fp64,
one token at a time, backward by back-propagation through time).  This module
only marshals CPU arrays into it.

Sources followed: the AMD ROCm blog "Pretraining hybrid LLMs with Primus",
section "How hybrid models are defined in Primus" (mixer list under Table 2):
Mamba2 decays its state with one scalar gate per head; Gated DeltaNet adds the
delta rule (the association of the current key is replaced, not only
accumulated) and keeps one scalar forget gate per head; Kimi Delta Attention
refines the gate to one value per key dimension.

Conventions: q, k, v, do are [B, T, H, d]; log_a and beta are [B, T, H]
(log_a is [B, T, H, d_k] for KDA); states are [B, H, d_k, d_v] (the transpose
of the d_v x d_k matrix S of the delta-rule recurrence); o_t reads the state
after token t's write.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
VARIANTS = {"gdn": 0, "ssd": 1, "kda": 2}

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b

            _b.build()
        lib = ctypes.CDLL(path)
        vp, dp, ci = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int
        lib.oracle_fwd.argtypes = [ci, vp, vp, vp, ci, vp, vp, vp, ci, dp, dp] + [ci] * 8
        lib.oracle_fwd.restype = ci
        lib.oracle_bwd.argtypes = [ci, vp, vp, vp, ci, vp, vp, vp, ci, vp, vp] + [dp] * 6 + [ci] * 6
        lib.oracle_bwd.restype = ci
        lib.oracle_max_threads.restype = ci
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _typed(x):
    """(pointer, dtype code, keepalive) for a CPU tensor/array of f32, bf16 or f64."""
    if x is None:
        return None, 0, None
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must be CPU tensors")
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x.data_ptr(), 1, x
        if x.dtype == torch.float32:
            return x.data_ptr(), 0, x
        if x.dtype == torch.float64:
            return x.data_ptr(), 2, x
        raise TypeError(f"unsupported dtype {x.dtype}")
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a.ctypes.data, 0, a
    if a.dtype == np.float64:
        return a.ctypes.data, 2, a
    raise TypeError(f"unsupported dtype {a.dtype}")


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def _shape(q, v):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    return int(B), int(T), int(H), int(dk), int(dv)


def _gates(variant, log_a, beta, h0, dht=None):
    """Gates, beta and states share one float type (f32 or f64)."""
    parts = [_typed(x) for x in (log_a, beta, h0, dht)]
    codes = {p[1] for p, x in zip(parts, (log_a, beta, h0, dht)) if x is not None}
    if len(codes) != 1 or 1 in codes:
        raise TypeError("log_a, beta, h0, dht must all be float32 or all float64")
    return parts, codes.pop()


def fwd(variant, q, k, v, log_a, beta=None, h0=None, cols=None, threads=0):
    """Forward of ``variant`` ('gdn', 'ssd', 'kda') in fp64.

    Returns (o [B,T,H,nc], ht [B,H,d_k,nc]) for value columns ``cols``
    (a (start, count) pair; default all columns).
    """
    var = VARIANTS[variant]
    B, T, H, dk, dv = _shape(q, v)
    c0, nc = (0, dv) if cols is None else (int(cols[0]), int(cols[1]))
    pq, dt, kq = _typed(q)
    pk, dt2, kk = _typed(k)
    pv, dt3, kv = _typed(v)
    if not (dt == dt2 == dt3):
        raise TypeError("q, k, v must share a dtype")
    if var == VARIANTS["ssd"]:
        beta = None
    parts, gdt = _gates(var, log_a, beta, h0)
    (pa, _, ka), (pb, _, kb), (ph, _, kh), _ = parts
    o = np.zeros((B, T, H, nc), np.float64)
    ht = np.zeros((B, H, dk, nc), np.float64)
    rc = _load().oracle_fwd(var, pq, pk, pv, dt, pa, pb, ph, gdt, _dptr(o), _dptr(ht),
                            B, T, H, dk, dv, c0, nc, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd failed with code {rc}")
    return o, ht


def bwd(variant, q, k, v, log_a, beta, h0, do, dht=None, threads=0):
    """Gradients (dq, dk, dv, dlog_a, dbeta, dh0) in fp64 of the loss
    <do, o> + <dht, ht> with respect to the inputs as passed."""
    var = VARIANTS[variant]
    B, T, H, dk, dv = _shape(q, v)
    pq, dt, kq = _typed(q)
    pk, _, kk = _typed(k)
    pv, _, kv = _typed(v)
    pd, dt4, kd = _typed(do)
    if dt4 != dt:
        raise TypeError("do must have the dtype of q, k, v")
    if var == VARIANTS["ssd"]:
        beta = None
    parts, gdt = _gates(var, log_a, beta, h0, dht)
    (pa, _, ka), (pb, _, kb), (ph, _, kh), (pt, _, kt) = parts
    dq = np.zeros((B, T, H, dk), np.float64)
    dkk = np.zeros((B, T, H, dk), np.float64)
    dvv = np.zeros((B, T, H, dv), np.float64)
    dla = np.zeros((B, T, H, dk) if var == VARIANTS["kda"] else (B, T, H), np.float64)
    db = np.zeros((B, T, H), np.float64)
    dh0 = np.zeros((B, H, dk, dv), np.float64)
    rc = _load().oracle_bwd(var, pq, pk, pv, dt, pa, pb, ph, gdt, pd, pt,
                            _dptr(dq), _dptr(dkk), _dptr(dvv), _dptr(dla), _dptr(db), _dptr(dh0),
                            B, T, H, dk, dv, int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed with code {rc}")
    return dq, dkk, dvv, dla, db, dh0
