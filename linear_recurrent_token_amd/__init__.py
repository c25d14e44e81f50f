"""Python binding of liblrt.so: gated delta-rule token mixers on MI355X.

Argument marshalling only.  Every step of every mixer runs in the library's
gfx950 kernels; this module checks tensors, allocates outputs and the
workspace with torch on the inputs' device, and passes raw pointers and the
current HIP stream through ctypes.  There is no CPU fallback: if the library
is missing, every call raises.

Entry points (names as in include/lrt.h):
  gdn_fwd(q, k, v, log_a, beta, h0=None, chunk=64)            -> (o, ht)
  gdn_bwd(q, k, v, log_a, beta, h0, do, dht=None, chunk=64)   -> (dq, dk, dv, dlog_a, dbeta, dh0)
  gdn_fwd_train(q, k, v, log_a, beta, h0=None, chunk=64)      -> (o, ht, saved)
  gdn_bwd_saved(q, k, v, log_a, beta, h0, do, saved, dht=None, chunk=64) -> as gdn_bwd
  gdn_fwd_noalloc(q, k, v, log_a, beta, h0=None, chunk=64)    -> (o, ht)   (static workspace)
  gdn_fwd_varlen / kda_fwd_varlen(q, k, v, log_a, beta, cu_seqlens, h0=None, chunk=64) -> (o, ht)
  gdn_fwd_fused / kda_fwd_fused(q_raw, k_raw, v, gate_raw, beta_raw, h0=None, chunk=64) -> (o, ht)
  gdn_bwd_varlen(q, k, v, log_a, beta, cu_seqlens, h0, do, dht=None, chunk=64) -> as gdn_bwd
  kda_fwd(q, k, v, log_a, beta, h0=None, chunk=64)            -> (o, ht)
  ssd_fwd(q, k, v, log_a, h0=None, chunk=64)                   -> (o, ht)
  ssd_bwd(q, k, v, log_a, h0, do, dht=None, chunk=64)          -> (dq, dk, dv, dlog_a, dh0)
  ssd_fwd_train(q, k, v, log_a, h0=None, chunk=64)             -> (o, ht, saved)
  ssd_bwd_saved(q, k, v, log_a, h0, do, saved, dht=None, chunk=64) -> as ssd_bwd
Layouts: q, k [B,T,H,d_k], v [B,T,H,d_v] (fp32 or bf16); log_a, beta fp32
[B,T,H] (KDA log_a [B,T,H,d_k]); states fp32 [B,H,d_k,d_v].
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblrt.so")

LRT_F32, LRT_BF16 = 0, 1
OP_GDN_FWD, OP_GDN_BWD, OP_KDA_FWD, OP_SSD_FWD, OP_SSD_BWD = 0, 1, 2, 3, 4
OP_GDN_FWD_VARLEN, OP_GDN_BWD_VARLEN, OP_KDA_FWD_VARLEN = 5, 6, 7
OP_KDA_BWD, OP_KDA_BWD_VARLEN = 8, 9
EXPORTS = ("gdn_fwd", "gdn_bwd", "gdn_fwd_train", "gdn_bwd_saved", "gdn_fwd_noalloc", "kda_fwd", "ssd_fwd",
           "ssd_bwd", "ssd_fwd_train", "ssd_bwd_saved", "gdn_fwd_varlen", "kda_fwd_varlen", "gdn_bwd_varlen",
           "gdn_fwd_fused", "kda_fwd_fused", "kda_bwd", "kda_bwd_varlen", "kda_fwd_train", "kda_bwd_saved",
           "kda_fwd_fused_lowrank", "short_conv_fwd", "short_conv_bwd", "short_conv_bwd_workspace_bytes",
           "gated_rmsnorm_fwd", "gated_rmsnorm_bwd", "gated_rmsnorm_bwd_workspace_bytes",
           "lrt_workspace_bytes", "lrt_status_string", "lrt_profile_attach", "lrt_profile_count",
           "lrt_kernel_name")
NOALLOC_MAX_BYTES = 64 << 20  # LRT_NOALLOC_MAX_BYTES

_lib = None


class LrtError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"liblrt.so not found at {LIB_PATH}; build it with "
                               "`python -m linear_recurrent_token_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.gdn_fwd.argtypes = [vp] * 8 + [ci] * 7 + [vp, sz, vp]
        L.kda_fwd.argtypes = [vp] * 8 + [ci] * 7 + [vp, sz, vp]
        L.ssd_fwd.argtypes = [vp] * 7 + [ci] * 7 + [vp, sz, vp]
        L.gdn_bwd.argtypes = [vp] * 14 + [ci] * 7 + [vp, sz, vp]
        L.ssd_bwd.argtypes = [vp] * 12 + [ci] * 7 + [vp, sz, vp]
        L.gdn_fwd_train.argtypes = [vp] * 8 + [ci] * 7 + [vp, sz, vp]
        L.gdn_bwd_saved.argtypes = [vp] * 14 + [ci] * 7 + [vp, sz, vp]
        L.ssd_fwd_train.argtypes = [vp] * 7 + [ci] * 7 + [vp, sz, vp]
        L.ssd_bwd_saved.argtypes = [vp] * 12 + [ci] * 7 + [vp, sz, vp]
        L.gdn_fwd_noalloc.argtypes = [vp] * 8 + [ci] * 7 + [vp]
        L.gdn_fwd_varlen.argtypes = [vp] * 9 + [ci] * 7 + [vp, sz, vp]
        L.kda_fwd_varlen.argtypes = [vp] * 9 + [ci] * 7 + [vp, sz, vp]
        L.gdn_bwd_varlen.argtypes = [vp] * 15 + [ci] * 7 + [vp, sz, vp]
        L.gdn_fwd_fused.argtypes = [vp] * 8 + [ci] * 7 + [vp, sz, vp]
        L.kda_fwd_fused.argtypes = [vp] * 8 + [ci] * 7 + [vp, sz, vp]
        L.kda_bwd.argtypes = [vp] * 14 + [ci] * 7 + [vp, sz, vp]
        L.kda_bwd_varlen.argtypes = [vp] * 15 + [ci] * 7 + [vp, sz, vp]
        L.kda_fwd_train.argtypes = [vp] * 8 + [ci] * 7 + [vp, sz, vp]
        L.kda_fwd_fused_lowrank.argtypes = [vp] * 5 + [ci] + [vp] * 4 + [ci] * 7 + [vp, sz, vp]
        L.kda_bwd_saved.argtypes = [vp] * 14 + [ci] * 7 + [vp, sz, vp]
        ll, cf = ctypes.c_longlong, ctypes.c_float
        L.short_conv_fwd.argtypes = [vp] * 4 + [ci] * 5 + [vp]
        L.short_conv_bwd.argtypes = [vp] * 6 + [ci] * 5 + [vp, sz, vp]
        L.short_conv_bwd_workspace_bytes.argtypes = [ll, ci, ci]
        L.short_conv_bwd_workspace_bytes.restype = sz
        L.gated_rmsnorm_fwd.argtypes = [vp] * 4 + [ll, ci, cf, ci, vp]
        L.gated_rmsnorm_bwd.argtypes = [vp] * 7 + [ll, ci, cf, ci, vp, sz, vp]
        L.gated_rmsnorm_bwd_workspace_bytes.argtypes = [ll, ci]
        L.gated_rmsnorm_bwd_workspace_bytes.restype = sz
        for f in ("short_conv_fwd", "short_conv_bwd", "gated_rmsnorm_fwd", "gated_rmsnorm_bwd"):
            getattr(L, f).restype = ci
        for f in ("gdn_fwd", "kda_fwd", "ssd_fwd", "gdn_bwd", "ssd_bwd", "gdn_fwd_train", "gdn_bwd_saved",
                  "ssd_fwd_train", "ssd_bwd_saved", "gdn_fwd_noalloc", "gdn_fwd_varlen", "kda_fwd_varlen",
                  "gdn_bwd_varlen", "gdn_fwd_fused", "kda_fwd_fused", "kda_bwd", "kda_bwd_varlen",
                  "kda_fwd_train", "kda_bwd_saved", "kda_fwd_fused_lowrank"):
            getattr(L, f).restype = ci
        L.lrt_workspace_bytes.argtypes = [ci] * 8
        L.lrt_workspace_bytes.restype = sz
        L.lrt_status_string.argtypes = [ci]
        L.lrt_status_string.restype = ctypes.c_char_p
        L.lrt_profile_attach.argtypes = [vp, vp, ci]
        L.lrt_profile_attach.restype = ci
        L.lrt_profile_count.restype = ci
        L.lrt_kernel_name.argtypes = [ci]
        L.lrt_kernel_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lrt_status_string(int(status)).decode()


def workspace_bytes(op, B, T, H, dk, dv, chunk, dtype) -> int:
    n = lib().lrt_workspace_bytes(op, B, T, H, dk, dv, chunk, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for lrt_workspace_bytes")
    return int(n)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return LRT_BF16
    if t.dtype == torch.float32:
        return LRT_F32
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _check(dev, dt, name, t, shape, dtype):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device != dev:
        raise ValueError(f"{name} must be a tensor on {dev}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(op, dev, B, T, H, dk, dv, chunk, dt, workspace):
    need = workspace_bytes(op, B, T, H, dk, dv, chunk, dt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace, need


def _fwd(fn, op, q, k, v, log_a, beta, h0, chunk, o, ht, workspace, kda=False, want_ws=False,
         gate_dtype=torch.float32):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    _check(dev, dt, "k", k, (B, T, H, dk), dt)
    _check(dev, dt, "v", v, (B, T, H, dv), dt)
    _check(dev, dt, "q", q, (B, T, H, dk), dt)
    _check(dev, dt, "log_a", log_a, (B, T, H, dk) if kda else (B, T, H), gate_dtype)
    ssd = fn.__name__.startswith("ssd")
    if not ssd:
        if beta is None:
            raise ValueError("beta is required")
        _check(dev, dt, "beta", beta, (B, T, H), torch.float32)
    _check(dev, dt, "h0", h0, (B, H, dk, dv), torch.float32)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(dev, dt, "o", o, (B, T, H, dv), dt)
    if ht is True:
        ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif ht is False:
        ht = None
    _check(dev, dt, "ht", ht, (B, H, dk, dv), torch.float32)
    code = _dtype_code(q)
    ws, need = _workspace(op, dev, B, T, H, dk, dv, chunk, code, workspace)
    with torch.cuda.device(dev):
        if ssd:
            rc = fn(_p(q), _p(k), _p(v), _p(log_a), _p(h0), _p(o), _p(ht), B, T, H, dk, dv, chunk, code,
                    _p(ws), need, _stream(dev))
        else:
            rc = fn(_p(q), _p(k), _p(v), _p(log_a), _p(beta), _p(h0), _p(o), _p(ht), B, T, H, dk, dv, chunk,
                    code, _p(ws), need, _stream(dev))
    if rc != 0:
        raise LrtError(fn.__name__, rc)
    return (o, ht, ws) if want_ws else (o, ht)


def gdn_fwd(q, k, v, log_a, beta, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Gated DeltaNet forward -> (o, ht).  ht=False skips the final state."""
    return _fwd(lib().gdn_fwd, OP_GDN_FWD, q, k, v, log_a, beta, h0, chunk, o, ht, workspace)


def gdn_fwd_train(q, k, v, log_a, beta, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Gated DeltaNet forward that keeps what the backward needs -> (o, ht,
    saved); pass ``saved`` (a uint8 workspace of the backward's size) to
    gdn_bwd_saved."""
    return _fwd(lib().gdn_fwd_train, OP_GDN_BWD, q, k, v, log_a, beta, h0, chunk, o, ht, workspace, want_ws=True)


def kda_fwd_train(q, k, v, log_a, beta, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Kimi Delta Attention forward that keeps what the backward needs ->
    (o, ht, saved); pass ``saved`` to kda_bwd_saved."""
    return _fwd(lib().kda_fwd_train, OP_KDA_BWD, q, k, v, log_a, beta, h0, chunk, o, ht, workspace, kda=True,
                want_ws=True)


def kda_bwd_saved(q, k, v, log_a, beta, h0, do, saved, dht=None, chunk=64, want_dh0=True, out=None):
    """Kimi Delta Attention backward from kda_fwd_train's ``saved`` workspace
    (no recompute) -> (dq, dk, dv, dlog_a, dbeta, dh0 or None)."""
    if saved is None:
        raise ValueError("saved: the workspace kda_fwd_train returned")
    return _bwd(True, q, k, v, log_a, beta, h0, do, dht, chunk, want_dh0, saved, out, fn="kda_bwd_saved")


def ssd_fwd_train(q, k, v, log_a, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Mamba2 forward that keeps the chunk-start states and gate cumsums ->
    (o, ht, saved) for ssd_bwd_saved."""
    return _fwd(lib().ssd_fwd_train, OP_SSD_BWD, q, k, v, log_a, None, h0, chunk, o, ht, workspace, want_ws=True)


def ssd_bwd_saved(q, k, v, log_a, h0, do, saved, dht=None, chunk=64, want_dh0=True, out=None):
    """Mamba2 backward from ssd_fwd_train's ``saved`` workspace -> (dq, dk,
    dv, dlog_a, dh0 or None)."""
    if saved is None:
        raise ValueError("saved: the workspace ssd_fwd_train returned")
    if out is not None:
        out = tuple(out[:4]) + (None,) + tuple(out[4:])
    g = _bwd(False, q, k, v, log_a, None, h0, do, dht, chunk, want_dh0, saved, out, fn="ssd_bwd_saved")
    return g[:4] + g[5:]


def gdn_bwd_saved(q, k, v, log_a, beta, h0, do, saved, dht=None, chunk=64, want_dh0=True, out=None):
    """Gated DeltaNet backward from gdn_fwd_train's ``saved`` workspace (no
    recompute) -> (dq, dk, dv, dlog_a, dbeta, dh0 or None)."""
    if saved is None:
        raise ValueError("saved: the workspace gdn_fwd_train returned")
    return _bwd(True, q, k, v, log_a, beta, h0, do, dht, chunk, want_dh0, saved, out, fn="gdn_bwd_saved")


def gdn_fwd_noalloc(q, k, v, log_a, beta, h0=None, chunk=64, o=None, ht=True):
    """gdn_fwd with the library's static per-GPU workspace (nothing is
    allocated by the library; pass preallocated o / ht to allocate nothing
    at all) -> (o, ht).  Sizes whose workspace exceeds NOALLOC_MAX_BYTES raise
    LrtError (LRT_ERR_TOO_LARGE)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    for name, t, shp, ty in (("k", k, (B, T, H, dk), dt), ("v", v, (B, T, H, dv), dt),
                             ("log_a", log_a, (B, T, H), torch.float32), ("beta", beta, (B, T, H), torch.float32),
                             ("h0", h0, (B, H, dk, dv), torch.float32)):
        _check(dev, dt, name, t, shp, ty)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(dev, dt, "o", o, (B, T, H, dv), dt)
    if ht is True:
        ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif ht is False:
        ht = None
    _check(dev, dt, "ht", ht, (B, H, dk, dv), torch.float32)
    with torch.cuda.device(dev):
        rc = lib().gdn_fwd_noalloc(_p(q), _p(k), _p(v), _p(log_a), _p(beta), _p(h0), _p(o), _p(ht), B, T, H, dk, dv,
                                   chunk, _dtype_code(q), _stream(dev))
    if rc != 0:
        raise LrtError("gdn_fwd_noalloc", rc)
    return o, ht


def gdn_fwd_fused(q_raw, k_raw, v, gate_raw, beta_raw, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Gated DeltaNet forward on the raw projections (q, k L2-normalised,
    beta = sigmoid(beta_raw), log a = -softplus(gate_raw), all inside the
    kernels) -> (o, ht).  gate_raw, beta_raw fp32 [B, T, H]."""
    return _fwd(lib().gdn_fwd_fused, OP_GDN_FWD, q_raw, k_raw, v, gate_raw, beta_raw, h0, chunk, o, ht, workspace)


def kda_fwd_fused(q_raw, k_raw, v, gate_raw, beta_raw, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Kimi Delta Attention forward on the raw projections -> (o, ht).
    gate_raw: the per-key-dimension gate pre-activation [B, T, H, d_k] in the
    dtype of q (log a = -softplus(gate_raw) inside the kernels)."""
    return _fwd(lib().kda_fwd_fused, OP_KDA_FWD, q_raw, k_raw, v, gate_raw, beta_raw, h0, chunk, o, ht, workspace,
                kda=True, gate_dtype=q_raw.dtype)


GATE_RANK = 16  # the rank of KDA's low-rank gate that kda_fwd_fused_lowrank takes


def kda_fwd_fused_lowrank(q_raw, k_raw, v, z, w_up, beta_raw, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Kimi Delta Attention forward on raw projections with the gate as its
    low-rank factors: z [B, T, 16] (each token's bottleneck activations) and
    w_up [H*d_k, 16], both in q's dtype; log a = -softplus(w_up z) is formed
    in the kernels -> (o, ht)."""
    B, T, H, dk = q_raw.shape
    dv = v.shape[-1]
    dev, dt = q_raw.device, q_raw.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    for name, t, shp, ty in (("k_raw", k_raw, (B, T, H, dk), dt), ("v", v, (B, T, H, dv), dt),
                             ("z", z, (B, T, GATE_RANK), dt), ("w_up", w_up, (H * dk, GATE_RANK), dt),
                             ("beta_raw", beta_raw, (B, T, H), torch.float32),
                             ("h0", h0, (B, H, dk, dv), torch.float32)):
        _check(dev, dt, name, t, shp, ty)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(dev, dt, "o", o, (B, T, H, dv), dt)
    if ht is True:
        ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif ht is False:
        ht = None
    _check(dev, dt, "ht", ht, (B, H, dk, dv), torch.float32)
    code = _dtype_code(q_raw)
    ws, need = _workspace(OP_KDA_FWD, dev, B, T, H, dk, dv, chunk, code, workspace)
    with torch.cuda.device(dev):
        rc = lib().kda_fwd_fused_lowrank(_p(q_raw), _p(k_raw), _p(v), _p(z), _p(w_up), GATE_RANK, _p(beta_raw),
                                         _p(h0), _p(o), _p(ht), B, T, H, dk, dv, chunk, code, _p(ws), need,
                                         _stream(dev))
    if rc != 0:
        raise LrtError("kda_fwd_fused_lowrank", rc)
    return o, ht


def _varlen_check(q, cu_seqlens):
    if q.shape[0] != 1:
        raise ValueError("packed sequences are laid out as [1, T, H, d]")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.device != q.device or \
            cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2 or \
            not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor [n_seq + 1] on the inputs' device")
    return cu_seqlens.numel() - 1


def _fwd_varlen(fn, op, q, k, v, log_a, beta, cu_seqlens, h0, chunk, kda):
    n = _varlen_check(q, cu_seqlens)
    _, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    for name, t, shp, ty in (("k", k, (1, T, H, dk), dt), ("v", v, (1, T, H, dv), dt),
                             ("log_a", log_a, (1, T, H, dk) if kda else (1, T, H), torch.float32),
                             ("beta", beta, (1, T, H), torch.float32), ("h0", h0, (n, H, dk, dv), torch.float32)):
        _check(dev, dt, name, t, shp, ty)
    o = torch.empty((1, T, H, dv), dtype=dt, device=dev)
    ht = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev)
    code = _dtype_code(q)
    ws, need = _workspace(op, dev, n, T, H, dk, dv, chunk, code, None)
    with torch.cuda.device(dev):
        rc = fn(_p(q), _p(k), _p(v), _p(log_a), _p(beta), _p(h0), _p(o), _p(ht), _p(cu_seqlens), n, T, H, dk, dv,
                chunk, code, _p(ws), need, _stream(dev))
    if rc != 0:
        raise LrtError(fn.__name__, rc)
    return o, ht


def gdn_fwd_varlen(q, k, v, log_a, beta, cu_seqlens, h0=None, chunk=64):
    """Gated DeltaNet forward over packed sequences (q [1, T, H, d_k], ...;
    cu_seqlens int32 [n_seq + 1]; h0 [n_seq, H, d_k, d_v] or None) -> (o, ht)."""
    return _fwd_varlen(lib().gdn_fwd_varlen, OP_GDN_FWD_VARLEN, q, k, v, log_a, beta, cu_seqlens, h0, chunk, False)


def kda_fwd_varlen(q, k, v, log_a, beta, cu_seqlens, h0=None, chunk=64):
    """Kimi Delta Attention forward over packed sequences -> (o, ht)."""
    return _fwd_varlen(lib().kda_fwd_varlen, OP_KDA_FWD_VARLEN, q, k, v, log_a, beta, cu_seqlens, h0, chunk, True)


def _bwd_varlen(fn, op, kda, q, k, v, log_a, beta, cu_seqlens, h0, do, dht, chunk, want_dh0):
    n = _varlen_check(q, cu_seqlens)
    _, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    gshape = (1, T, H, dk) if kda else (1, T, H)
    for name, t, shp, ty in (("k", k, (1, T, H, dk), dt), ("v", v, (1, T, H, dv), dt),
                             ("log_a", log_a, gshape, torch.float32), ("beta", beta, (1, T, H), torch.float32),
                             ("h0", h0, (n, H, dk, dv), torch.float32), ("do", do, (1, T, H, dv), dt),
                             ("dht", dht, (n, H, dk, dv), torch.float32)):
        _check(dev, dt, name, t, shp, ty)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    gla = torch.empty(gshape, dtype=torch.float32, device=dev)
    gb = torch.empty((1, T, H), dtype=torch.float32, device=dev)
    gh0 = torch.empty((n, H, dk, dv), dtype=torch.float32, device=dev) if want_dh0 else None
    code = _dtype_code(q)
    ws, need = _workspace(op, dev, n, T, H, dk, dv, chunk, code, None)
    with torch.cuda.device(dev):
        rc = fn(_p(q), _p(k), _p(v), _p(log_a), _p(beta), _p(h0), _p(do), _p(dht), _p(gq), _p(gk), _p(gv), _p(gla),
                _p(gb), _p(gh0), _p(cu_seqlens), n, T, H, dk, dv, chunk, code, _p(ws), need, _stream(dev))
    if rc != 0:
        raise LrtError(fn.__name__, rc)
    return gq, gk, gv, gla, gb, gh0


def gdn_bwd_varlen(q, k, v, log_a, beta, cu_seqlens, h0, do, dht=None, chunk=64, want_dh0=True):
    """Gated DeltaNet backward over packed sequences -> (dq, dk, dv, dlog_a,
    dbeta, dh0 [n_seq, H, d_k, d_v] or None)."""
    return _bwd_varlen(lib().gdn_bwd_varlen, OP_GDN_BWD_VARLEN, False, q, k, v, log_a, beta, cu_seqlens, h0, do, dht,
                       chunk, want_dh0)


def kda_bwd_varlen(q, k, v, log_a, beta, cu_seqlens, h0, do, dht=None, chunk=64, want_dh0=True):
    """Kimi Delta Attention backward over packed sequences -> (dq, dk, dv,
    dlog_a [1, T, H, d_k], dbeta, dh0 [n_seq, H, d_k, d_v] or None)."""
    return _bwd_varlen(lib().kda_bwd_varlen, OP_KDA_BWD_VARLEN, True, q, k, v, log_a, beta, cu_seqlens, h0, do, dht,
                       chunk, want_dh0)


def kda_fwd(q, k, v, log_a, beta, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Kimi Delta Attention forward (log_a per key dim) -> (o, ht)."""
    return _fwd(lib().kda_fwd, OP_KDA_FWD, q, k, v, log_a, beta, h0, chunk, o, ht, workspace, kda=True)


def ssd_fwd(q, k, v, log_a, h0=None, chunk=64, o=None, ht=True, workspace=None):
    """Mamba2 / SSD forward (no beta, no delta term) -> (o, ht)."""
    return _fwd(lib().ssd_fwd, OP_SSD_FWD, q, k, v, log_a, None, h0, chunk, o, ht, workspace)


def gdn_bwd(q, k, v, log_a, beta, h0, do, dht=None, chunk=64, want_dh0=True, workspace=None, out=None):
    """Gated DeltaNet backward -> (dq, dk, dv, dlog_a, dbeta, dh0 or None)."""
    return _bwd(True, q, k, v, log_a, beta, h0, do, dht, chunk, want_dh0, workspace, out)


def kda_bwd(q, k, v, log_a, beta, h0, do, dht=None, chunk=64, want_dh0=True, workspace=None, out=None):
    """Kimi Delta Attention backward (log_a and dlog_a per key dimension,
    [B, T, H, d_k]) -> (dq, dk, dv, dlog_a, dbeta, dh0 or None)."""
    return _bwd(True, q, k, v, log_a, beta, h0, do, dht, chunk, want_dh0, workspace, out, fn="kda_bwd")


def ssd_bwd(q, k, v, log_a, h0, do, dht=None, chunk=64, want_dh0=True, workspace=None, out=None):
    """Mamba2 / SSD backward -> (dq, dk, dv, dlog_a, dh0 or None)."""
    if out is not None:
        out = tuple(out[:4]) + (None,) + tuple(out[4:])
    g = _bwd(False, q, k, v, log_a, None, h0, do, dht, chunk, want_dh0, workspace, out)
    return g[:4] + g[5:]


def _bwd(delta, q, k, v, log_a, beta, h0, do, dht, chunk, want_dh0, workspace, out, fn="gdn_bwd"):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    kda = fn.startswith("kda")
    gshape = (B, T, H, dk) if kda else (B, T, H)
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    for name, t, shp, ty in (("k", k, (B, T, H, dk), dt), ("v", v, (B, T, H, dv), dt),
                             ("log_a", log_a, gshape, torch.float32),
                             ("beta", beta if delta else None, (B, T, H), torch.float32),
                             ("h0", h0, (B, H, dk, dv), torch.float32),
                             ("do", do, (B, T, H, dv), dt), ("dht", dht, (B, H, dk, dv), torch.float32)):
        _check(dev, dt, name, t, shp, ty)
    _check(dev, dt, "q", q, (B, T, H, dk), dt)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
               torch.empty(gshape, dtype=torch.float32, device=dev),
               torch.empty((B, T, H), dtype=torch.float32, device=dev) if delta else None,
               torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dh0 else None)
    gq, gk, gv, gla, gb, gh0 = out
    code = _dtype_code(q)
    op = OP_KDA_BWD if kda else OP_GDN_BWD if delta else OP_SSD_BWD
    ws, need = _workspace(op, dev, B, T, H, dk, dv, chunk, code, workspace)
    with torch.cuda.device(dev):
        if delta:
            rc = getattr(lib(), fn)(_p(q), _p(k), _p(v), _p(log_a), _p(beta), _p(h0), _p(do), _p(dht), _p(gq),
                                    _p(gk), _p(gv), _p(gla), _p(gb), _p(gh0), B, T, H, dk, dv, chunk, code, _p(ws),
                                    need, _stream(dev))
        else:
            fs = "ssd_bwd_saved" if fn.endswith("_saved") else "ssd_bwd"
            rc = getattr(lib(), fs)(_p(q), _p(k), _p(v), _p(log_a), _p(h0), _p(do), _p(dht), _p(gq), _p(gk),
                                    _p(gv), _p(gla), _p(gh0), B, T, H, dk, dv, chunk, code, _p(ws), need,
                                    _stream(dev))
            fn = fs
    if rc != 0:
        raise LrtError(fn, rc)
    return gq, gk, gv, gla, gb, gh0


# ------------------------------------------------------------------------
# The steps either side of the mixer: short convolution (+ SiLU) on its
# q/k/v projections and gated RMSNorm on its output (lrt.h documents them).

def _conv_args(x, w, cu_seqlens):
    if x.device.type != "cuda" or x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, T, D] tensor on a GPU device")
    B, T, D = x.shape
    if w.dtype != torch.float32 or w.device != x.device or w.dim() != 2 or w.shape[0] != D or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 [D, W] tensor on x's device")
    if cu_seqlens is None:
        return B, T, D, int(w.shape[1]), None
    if B != 1:
        raise ValueError("packed sequences take x as [1, T, D]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != x.device or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be an int32 vector on x's device")
    return int(cu_seqlens.numel()) - 1, T, D, int(w.shape[1]), cu_seqlens


def short_conv(x, w, cu_seqlens=None, out=None):
    """silu(causal depthwise conv(x, w)) per sequence: x [B, T, D] (or packed
    [1, T, D] with cu_seqlens), w [D, W] float32.  Returns y like x."""
    n, T, D, W, cu = _conv_args(x, w, cu_seqlens)
    y = torch.empty_like(x) if out is None else out
    _check(x.device, x.dtype, "out", y, tuple(x.shape), x.dtype)
    rc = lib().short_conv_fwd(_p(x), _p(w), _p(y), _p(cu), n, T, D, W, _dtype_code(x), _stream(x.device))
    if rc != 0:
        raise LrtError("short_conv_fwd", rc)
    return y


def short_conv_bwd(x, w, dy, cu_seqlens=None, workspace=None):
    """(dx, dw) of sum(dy * short_conv(x, w)); dw float32 [D, W]."""
    n, T, D, W, cu = _conv_args(x, w, cu_seqlens)
    _check(x.device, x.dtype, "dy", dy, tuple(x.shape), x.dtype)
    need = int(lib().short_conv_bwd_workspace_bytes(x.shape[0] * T, D, W))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x)
    dw = torch.empty((D, W), dtype=torch.float32, device=x.device)
    rc = lib().short_conv_bwd(_p(x), _p(w), _p(dy), _p(dx), _p(dw), _p(cu), n, T, D, W, _dtype_code(x),
                              _p(workspace), workspace.numel() * workspace.element_size(), _stream(x.device))
    if rc != 0:
        raise LrtError("short_conv_bwd", rc)
    return dx, dw


def _norm_args(o, z, w):
    if o.device.type != "cuda" or not o.is_contiguous():
        raise ValueError("o must be a contiguous tensor on a GPU device")
    d = int(o.shape[-1])
    _check(o.device, o.dtype, "z", z, tuple(o.shape), o.dtype)
    _check(o.device, o.dtype, "w", w, (d,), torch.float32)
    return o.numel() // d if d else 0, d


def gated_rmsnorm(o, z, w, eps=1e-6):
    """o / sqrt(mean(o^2) + eps) * w * silu(z) over the last axis; w float32 [d]."""
    rows, d = _norm_args(o, z, w)
    y = torch.empty_like(o)
    rc = lib().gated_rmsnorm_fwd(_p(o), _p(z), _p(w), _p(y), rows, d, float(eps), _dtype_code(o),
                                 _stream(o.device))
    if rc != 0:
        raise LrtError("gated_rmsnorm_fwd", rc)
    return y


def gated_rmsnorm_bwd(o, z, w, dy, eps=1e-6, workspace=None):
    """(do, dz, dw) of sum(dy * gated_rmsnorm(o, z, w)); dw float32 [d]."""
    rows, d = _norm_args(o, z, w)
    _check(o.device, o.dtype, "dy", dy, tuple(o.shape), o.dtype)
    need = int(lib().gated_rmsnorm_bwd_workspace_bytes(rows, d))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=o.device)
    do, dz = torch.empty_like(o), torch.empty_like(o)
    dw = torch.empty((d,), dtype=torch.float32, device=o.device)
    rc = lib().gated_rmsnorm_bwd(_p(o), _p(z), _p(w), _p(dy), _p(do), _p(dz), _p(dw), rows, d, float(eps),
                                 _dtype_code(o), _p(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(o.device))
    if rc != 0:
        raise LrtError("gated_rmsnorm_bwd", rc)
    return do, dz, dw
