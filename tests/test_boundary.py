"""The C ABI boundary on the CPU: liblrt.so loads, exports every function
include/lrt.h declares, and rejects invalid arguments with the documented
status codes before touching the GPU (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrt.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def codes():
    src = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"#define\s+(LRT_\w+)\s+\(?(-?\d+)\)?", src)}


@pytest.fixture(scope="module")
def L():
    import linear_recurrent_token_amd as L
    return L


def test_header_declares_the_entry_points():
    names = declared()
    for f in ("gdn_fwd", "gdn_bwd", "kda_fwd", "ssd_fwd", "ssd_bwd", "lrt_workspace_bytes", "lrt_status_string"):
        assert f in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    for name in declared():
        assert hasattr(lib, name), name
    assert set(L.EXPORTS) == set(declared())


def test_status_codes_match_header(L):
    c = codes()
    assert c["LRT_OK"] == 0
    for name in ("LRT_ERR_NULL", "LRT_ERR_SHAPE", "LRT_ERR_CHUNK", "LRT_ERR_DTYPE", "LRT_ERR_WORKSPACE",
                 "LRT_ERR_ALIGN", "LRT_ERR_LAUNCH", "LRT_ERR_OP"):
        assert c[name] < 0
        s = L.status_string(c[name])
        assert s and s != "unknown status"
    assert L.status_string(12345) == "unknown status"


def _fwd(L, fn="gdn_fwd", q=None, k=None, v=None, la=None, b=None, h0=None, o=None, ht=None, B=1, T=64, H=2,
         dk=16, dv=16, chunk=16, dtype=0, ws=None, wsb=0):
    lib = L.lib()
    args = [q, k, v, la] + ([b] if fn != "ssd_fwd" else []) + [h0, o, ht, B, T, H, dk, dv, chunk, dtype, ws, wsb,
                                                               None]
    return getattr(lib, fn)(*args)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def test_validation_errors_before_any_launch(L):
    c = codes()
    ok = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE, o=FAKE)
    assert _fwd(L, dtype=7, **ok) == c["LRT_ERR_DTYPE"]
    assert _fwd(L, dk=48, **ok) == c["LRT_ERR_SHAPE"]
    assert _fwd(L, dv=256, **ok) == c["LRT_ERR_SHAPE"]
    assert _fwd(L, B=0, **ok) == c["LRT_ERR_SHAPE"]
    assert _fwd(L, T=-1, **ok) == c["LRT_ERR_SHAPE"]
    assert _fwd(L, chunk=128, **ok) == c["LRT_ERR_CHUNK"]
    assert _fwd(L, chunk=8, **ok) == c["LRT_ERR_CHUNK"]
    # a chunk tile's offsets must fit 32 bits: H * max(d_k, d_v) < 2^24
    assert _fwd(L, H=1 << 17, dk=128, dv=16, **ok) == c["LRT_ERR_SHAPE"]
    assert _fwd(L, H=(1 << 17) - 1, dk=128, dv=16, **ok) == c["LRT_ERR_WORKSPACE"]
    for missing in ("q", "k", "v", "la", "b", "o"):
        a = dict(ok)
        a[missing] = None
        assert _fwd(L, **a) == c["LRT_ERR_NULL"], missing
    a = dict(ok)
    a["q"] = FAKE + 8
    assert _fwd(L, **a) == c["LRT_ERR_ALIGN"]
    a = dict(ok)
    a["la"] = FAKE + 2
    assert _fwd(L, **a) == c["LRT_ERR_ALIGN"]
    a = dict(ok)
    a["la"] = FAKE + 4  # gates need only 4-byte alignment
    assert _fwd(L, **a) == c["LRT_ERR_WORKSPACE"]
    need = L.workspace_bytes(L.OP_GDN_FWD, 1, 64, 2, 16, 16, 16, 0)
    assert _fwd(L, ws=FAKE, wsb=need - 1, **ok) == c["LRT_ERR_WORKSPACE"]
    # SSD does not need beta
    assert _fwd(L, fn="ssd_fwd", **ok) == c["LRT_ERR_WORKSPACE"]


def test_backward_validation(L):
    c = codes()
    lib = L.lib()
    F = FAKE
    base = [F, F, F, F, F, None, F, None, F, F, F, F, F, None, 1, 64, 2, 16, 16, 16, 0, None, 0, None]
    assert lib.gdn_bwd(*base) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):
        a = list(base)
        a[i] = None
        assert lib.gdn_bwd(*a) == c["LRT_ERR_NULL"], i
    a = list(base)
    a[19] = 48
    assert lib.gdn_bwd(*a) == c["LRT_ERR_CHUNK"]
    a[19] = 32  # a valid chunk: validation gets as far as the (missing) workspace
    assert lib.gdn_bwd(*a) == c["LRT_ERR_WORKSPACE"]
    a = list(base)
    a[20] = 2
    assert lib.gdn_bwd(*a) == c["LRT_ERR_DTYPE"]


def test_training_pair_validation(L):
    c = codes()
    lib = L.lib()
    F = FAKE
    # gdn_fwd_train needs the backward's workspace, not the forward's
    fwd_need = L.workspace_bytes(L.OP_GDN_FWD, 1, 64, 2, 16, 16, 16, 0)
    bwd_need = L.workspace_bytes(L.OP_GDN_BWD, 1, 64, 2, 16, 16, 16, 0)
    assert bwd_need > fwd_need
    args = [F, F, F, F, F, None, F, None, 1, 64, 2, 16, 16, 16, 0, F, fwd_need, None]
    assert lib.gdn_fwd_train(*args) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 4, 6):
        a = list(args)
        a[i] = None
        assert lib.gdn_fwd_train(*a) == c["LRT_ERR_NULL"], i
    # fp32 at d_k = d_v = 128 is accepted (the kernels run a chunk that fits
    # in LDS); a too-small workspace is still rejected before any launch
    need128 = L.workspace_bytes(L.OP_GDN_BWD, 1, 64, 2, 128, 128, 64, 0)
    assert 0 < need128 < (1 << 40)
    a = list(args)
    a[11], a[12], a[13], a[16] = 128, 128, 64, need128 - 1
    assert lib.gdn_fwd_train(*a) == c["LRT_ERR_WORKSPACE"]
    base = [F, F, F, F, F, None, F, None, F, F, F, F, F, None, 1, 64, 2, 16, 16, 16, 0, None, 0, None]
    assert lib.gdn_bwd_saved(*base) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):
        a = list(base)
        a[i] = None
        assert lib.gdn_bwd_saved(*a) == c["LRT_ERR_NULL"], i


def test_ssd_training_pair_validation(L):
    c = codes()
    lib = L.lib()
    F = FAKE
    fwd_need = L.workspace_bytes(L.OP_SSD_FWD, 1, 64, 2, 16, 16, 16, 0)
    bwd_need = L.workspace_bytes(L.OP_SSD_BWD, 1, 64, 2, 16, 16, 16, 0)
    assert bwd_need > fwd_need
    # q k v log_a h0 o ht | B T H dk dv chunk dtype | ws wsb stream
    args = [F, F, F, F, None, F, None, 1, 64, 2, 16, 16, 16, 0, F, fwd_need, None]
    assert lib.ssd_fwd_train(*args) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 5):
        a = list(args)
        a[i] = None
        assert lib.ssd_fwd_train(*a) == c["LRT_ERR_NULL"], i
    # fp32 at d = 128 is accepted; a too-small workspace is rejected before any launch
    need128 = L.workspace_bytes(L.OP_SSD_BWD, 1, 64, 2, 128, 128, 64, 0)
    a = list(args)
    a[10], a[11], a[12], a[15] = 128, 128, 64, need128 - 1
    assert lib.ssd_fwd_train(*a) == c["LRT_ERR_WORKSPACE"]
    base = [F, F, F, F, None, F, None, F, F, F, F, None, 1, 64, 2, 16, 16, 16, 0, None, 0, None]
    assert lib.ssd_bwd_saved(*base) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 5, 7, 8, 9, 10):
        a = list(base)
        a[i] = None
        assert lib.ssd_bwd_saved(*a) == c["LRT_ERR_NULL"], i


def test_ssd_backward_validation(L):
    c = codes()
    lib = L.lib()
    F = FAKE
    # q k v log_a h0 do dht dq dk dv dlog_a dh0 | B T H dk dv chunk dtype | ws wsb stream
    base = [F, F, F, F, None, F, None, F, F, F, F, None, 1, 64, 2, 16, 16, 16, 0, None, 0, None]
    assert lib.ssd_bwd(*base) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 5, 7, 8, 9, 10):
        a = list(base)
        a[i] = None
        assert lib.ssd_bwd(*a) == c["LRT_ERR_NULL"], i
    a = list(base)
    a[17] = 48
    assert lib.ssd_bwd(*a) == c["LRT_ERR_CHUNK"]
    a = list(base)
    a[18] = 2
    assert lib.ssd_bwd(*a) == c["LRT_ERR_DTYPE"]
    a = list(base)
    a[15] = 24
    assert lib.ssd_bwd(*a) == c["LRT_ERR_SHAPE"]
    a = list(base)
    a[3] = F + 2
    assert lib.ssd_bwd(*a) == c["LRT_ERR_ALIGN"]
    need = L.workspace_bytes(L.OP_SSD_BWD, 1, 64, 2, 16, 16, 16, 0)
    a = list(base)
    a[19], a[20] = F, need - 1
    assert lib.ssd_bwd(*a) == c["LRT_ERR_WORKSPACE"]


def test_workspace_bytes(L):
    lib = L.lib()
    bad = ctypes.c_size_t(-1).value
    assert lib.lrt_workspace_bytes(11, 1, 64, 2, 16, 16, 16, 0) == bad
    assert lib.lrt_workspace_bytes(10, 1, 64, 2, 16, 16, 16, 0) == bad
    assert lib.lrt_workspace_bytes(-1, 1, 64, 2, 16, 16, 16, 0) == bad
    assert lib.lrt_workspace_bytes(0, 1, 64, 2, 16, 16, 17, 0) == bad
    for op in range(5):
        n = L.workspace_bytes(op, 16, 2048, 8, 128, 128, 64, 1)
        assert n > 0
    # grows with T and is never zero
    assert L.workspace_bytes(0, 1, 0, 1, 16, 16, 16, 0) > 0
    assert L.workspace_bytes(0, 1, 4096, 1, 16, 16, 16, 0) > L.workspace_bytes(0, 1, 64, 1, 16, 16, 16, 0)
    # the backward needs more than the forward (Gated DeltaNet, KDA)
    assert L.workspace_bytes(1, 2, 256, 2, 64, 64, 64, 1) > L.workspace_bytes(0, 2, 256, 2, 64, 64, 64, 1)
    assert L.workspace_bytes(8, 2, 256, 2, 64, 64, 64, 1) > L.workspace_bytes(2, 2, 256, 2, 64, 64, 64, 1)
    # the fused Mamba2 forward needs none beyond the minimum
    assert L.workspace_bytes(3, 16, 2048, 8, 128, 128, 64, 1) == 256
    # every dtype and size of the supported set has a workspace (fp32 at
    # d = 128 runs a smaller chunk: its workspace is sized for that chunk)
    for op in range(10):
        for dt in (0, 1):
            for dk in (16, 32, 64, 128):
                for dv in (16, 32, 64, 128):
                    for ch in (16, 32, 64):
                        assert 0 < L.workspace_bytes(op, 2, 100, 2, dk, dv, ch, dt) < (1 << 40)


def test_python_binding_rejects_cpu_tensors(L):
    import torch
    x = torch.zeros((1, 8, 1, 16))
    with pytest.raises(ValueError):
        L.gdn_fwd(x, x, x, torch.zeros((1, 8, 1)), torch.zeros((1, 8, 1)))


def test_varlen_validation(L):
    """Packed-sequence entry points: cu_seqlens required and 4-byte aligned,
    n_seq >= 1, workspace of the packed op code; all before any launch."""
    c = codes()
    lib = L.lib()
    F = FAKE
    n, T, H, d, ch = 3, 100, 2, 16, 16
    need = L.workspace_bytes(L.OP_GDN_FWD_VARLEN, n, T, H, d, d, ch, 0)
    # the packed layout reserves room for a partial chunk per sequence
    assert need > L.workspace_bytes(L.OP_GDN_FWD, 1, T, H, d, d, ch, 0)
    # q k v log_a beta h0 o ht cu | n T H dk dv chunk dtype | ws wsb stream
    args = [F, F, F, F, F, None, F, None, F, n, T, H, d, d, ch, 0, F, need - 1, None]
    for fn in ("gdn_fwd_varlen", "kda_fwd_varlen"):
        f = getattr(lib, fn)
        assert f(*args) == c["LRT_ERR_WORKSPACE"], fn
        a = list(args)
        a[8] = None
        assert f(*a) == c["LRT_ERR_NULL"], fn
        a = list(args)
        a[8] = F + 2
        assert f(*a) == c["LRT_ERR_ALIGN"], fn
        a = list(args)
        a[9] = 0
        assert f(*a) == c["LRT_ERR_SHAPE"], fn
        a = list(args)
        a[14] = 48
        assert f(*a) == c["LRT_ERR_CHUNK"], fn
    bneed = L.workspace_bytes(L.OP_GDN_BWD_VARLEN, n, T, H, d, d, ch, 0)
    # q k v log_a beta h0 do dht dq dk dv dlog_a dbeta dh0 cu | n T H dk dv chunk dtype | ws wsb stream
    b = [F, F, F, F, F, None, F, None, F, F, F, F, F, None, F, n, T, H, d, d, ch, 0, F, bneed - 1, None]
    assert lib.gdn_bwd_varlen(*b) == c["LRT_ERR_WORKSPACE"]
    a = list(b)
    a[14] = None
    assert lib.gdn_bwd_varlen(*a) == c["LRT_ERR_NULL"]
    for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):
        a = list(b)
        a[i] = None
        assert lib.gdn_bwd_varlen(*a) == c["LRT_ERR_NULL"], i


def test_kda_backward_and_training_pair_validation(L):
    """kda_bwd, kda_bwd_saved, kda_fwd_train and kda_fwd_fused_lowrank reject
    missing pointers, bad sizes and short workspaces before any launch."""
    c = codes()
    lib = L.lib()
    F = FAKE
    base = [F, F, F, F, F, None, F, None, F, F, F, F, F, None, 1, 64, 2, 16, 16, 16, 0, None, 0, None]
    for fn in (lib.kda_bwd, lib.kda_bwd_saved):
        assert fn(*base) == c["LRT_ERR_WORKSPACE"]
        for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):
            a = list(base)
            a[i] = None
            assert fn(*a) == c["LRT_ERR_NULL"], i
        a = list(base)
        a[17] = 24
        assert fn(*a) == c["LRT_ERR_SHAPE"]
    # the KDA training forward needs the KDA backward's workspace, which holds
    # more than the forward's
    fwd_need = L.workspace_bytes(L.OP_KDA_FWD, 1, 64, 2, 16, 16, 16, 0)
    bwd_need = L.workspace_bytes(L.OP_KDA_BWD, 1, 64, 2, 16, 16, 16, 0)
    assert bwd_need > fwd_need
    args = [F, F, F, F, F, None, F, None, 1, 64, 2, 16, 16, 16, 0, F, fwd_need, None]
    assert lib.kda_fwd_train(*args) == c["LRT_ERR_WORKSPACE"]
    for i in (0, 1, 2, 3, 4, 6):
        a = list(args)
        a[i] = None
        assert lib.kda_fwd_train(*a) == c["LRT_ERR_NULL"], i
    # the low-rank gate: rank 16 only, W_up required, 16-byte aligned factors
    need = L.workspace_bytes(L.OP_KDA_FWD, 1, 64, 2, 16, 16, 16, 1)
    lr = [F, F, F, F, F, 16, F, None, F, None, 1, 64, 2, 16, 16, 16, 1, F, need, None]
    a = list(lr)
    a[5] = 8
    assert lib.kda_fwd_fused_lowrank(*a) == c["LRT_ERR_SHAPE"]
    a = list(lr)
    a[4] = None
    assert lib.kda_fwd_fused_lowrank(*a) == c["LRT_ERR_NULL"]
    a = list(lr)
    a[4] = FAKE + 2
    assert lib.kda_fwd_fused_lowrank(*a) == c["LRT_ERR_ALIGN"]
    a = list(lr)
    a[18] = need - 1
    assert lib.kda_fwd_fused_lowrank(*a) == c["LRT_ERR_WORKSPACE"]


def test_conv_and_gated_norm_validation(L):
    """short_conv_* and gated_rmsnorm_*: every invalid argument is rejected
    before a launch (each call below fails validation, so nothing runs)."""
    c = codes()
    lib = L.lib()
    F = FAKE
    SZ = ctypes.c_size_t(-1).value
    # short_conv_fwd(x, w, y, cu, n_seq, T, D, W, dtype, stream)
    conv = lambda x=F, w=F, y=F + 4096, cu=None, n=2, T=8, D=64, W=4, dt=1: lib.short_conv_fwd(
        x, w, y, cu, n, T, D, W, dt, None)
    assert conv(dt=7) == c["LRT_ERR_DTYPE"]
    assert conv(D=12) == c["LRT_ERR_SHAPE"]
    assert conv(D=0) == c["LRT_ERR_SHAPE"]
    assert conv(W=5) == c["LRT_ERR_SHAPE"]
    assert conv(W=1) == c["LRT_ERR_SHAPE"]
    assert conv(n=0) == c["LRT_ERR_SHAPE"]
    assert conv(T=-1) == c["LRT_ERR_SHAPE"]
    assert conv(x=None) == c["LRT_ERR_NULL"]
    assert conv(w=None) == c["LRT_ERR_NULL"]
    assert conv(y=None) == c["LRT_ERR_NULL"]
    assert conv(x=F + 8) == c["LRT_ERR_ALIGN"]
    assert conv(y=F + 8) == c["LRT_ERR_ALIGN"]
    assert conv(w=F + 2) == c["LRT_ERR_ALIGN"]
    assert conv(cu=F + 2) == c["LRT_ERR_ALIGN"]
    assert conv(y=F) == c["LRT_ERR_SHAPE"]  # in place
    assert conv(T=0) == c["LRT_OK"]  # no tokens: nothing to do, nothing launched
    # short_conv_bwd(x, w, dy, dx, dw, cu, n_seq, T, D, W, dtype, ws, ws_bytes, stream)
    need = lib.short_conv_bwd_workspace_bytes(16, 64, 4)
    assert need != SZ and need >= 256
    cb = lambda x=F, w=F, dy=F + 4096, dx=F + 8192, dw=F, cu=None, n=2, T=8, D=64, W=4, dt=1, ws=F, wsb=need: \
        lib.short_conv_bwd(x, w, dy, dx, dw, cu, n, T, D, W, dt, ws, wsb, None)
    assert cb(wsb=need - 1) == c["LRT_ERR_WORKSPACE"]
    assert cb(ws=None) == c["LRT_ERR_WORKSPACE"]
    assert cb(ws=F + 8) == c["LRT_ERR_WORKSPACE"]
    assert cb(dw=None) == c["LRT_ERR_NULL"]
    assert cb(dx=None) == c["LRT_ERR_NULL"]
    assert cb(dy=None) == c["LRT_ERR_NULL"]
    assert cb(dw=F + 2) == c["LRT_ERR_ALIGN"]
    assert cb(dx=F + 8) == c["LRT_ERR_ALIGN"]
    assert cb(dx=F + 4096) == c["LRT_ERR_SHAPE"]  # dx aliases dy
    assert cb(D=20) == c["LRT_ERR_SHAPE"]
    for bad in ((-1, 64, 4), (16, 12, 4), (16, 64, 5), (1 << 31, 64, 4)):
        assert lib.short_conv_bwd_workspace_bytes(*bad) == SZ, bad
    # gated_rmsnorm_fwd(o, z, w, y, rows, d, eps, dtype, stream)
    gn = lambda o=F, z=F + 4096, w=F, y=F + 8192, rows=10, d=128, eps=1e-6, dt=1: lib.gated_rmsnorm_fwd(
        o, z, w, y, rows, d, eps, dt, None)
    assert gn(dt=3) == c["LRT_ERR_DTYPE"]
    assert gn(d=48) == c["LRT_ERR_SHAPE"]
    assert gn(d=512) == c["LRT_ERR_SHAPE"]
    assert gn(rows=-1) == c["LRT_ERR_SHAPE"]
    assert gn(eps=-1.0) == c["LRT_ERR_SHAPE"]
    assert gn(eps=float("nan")) == c["LRT_ERR_SHAPE"]
    assert gn(o=None) == c["LRT_ERR_NULL"]
    assert gn(z=None) == c["LRT_ERR_NULL"]
    assert gn(w=None) == c["LRT_ERR_NULL"]
    assert gn(y=None) == c["LRT_ERR_NULL"]
    assert gn(o=F + 8) == c["LRT_ERR_ALIGN"]
    assert gn(w=F + 2) == c["LRT_ERR_ALIGN"]
    assert gn(y=F) == c["LRT_ERR_SHAPE"]  # y aliases o
    assert gn(rows=0) == c["LRT_OK"]
    # gated_rmsnorm_bwd(o, z, w, dy, do, dz, dw, rows, d, eps, dtype, ws, ws_bytes, stream)
    nneed = lib.gated_rmsnorm_bwd_workspace_bytes(10, 128)
    assert nneed != SZ and nneed > 0
    gb = lambda o=F, z=F + 4096, w=F, dy=F + 8192, do=F + 12288, dz=F + 16384, dw=F, rows=10, d=128, ws=F, \
        wsb=nneed: lib.gated_rmsnorm_bwd(o, z, w, dy, do, dz, dw, rows, d, 1e-6, 1, ws, wsb, None)
    assert gb(wsb=nneed - 1) == c["LRT_ERR_WORKSPACE"]
    assert gb(ws=None) == c["LRT_ERR_WORKSPACE"]
    assert gb(dw=None) == c["LRT_ERR_NULL"]
    assert gb(do=None) == c["LRT_ERR_NULL"]
    assert gb(dz=F + 12288) == c["LRT_ERR_SHAPE"]  # dz aliases do
    assert gb(do=F) == c["LRT_ERR_SHAPE"]  # do aliases o
    assert gb(dz=F + 8) == c["LRT_ERR_ALIGN"]
    assert lib.gated_rmsnorm_bwd_workspace_bytes(10, 100) == SZ
    assert lib.gated_rmsnorm_bwd_workspace_bytes(-5, 128) == SZ


def test_autograd_bindings_refuse_cpu_tensors(L):
    """The autograd layer is marshalling only: CPU tensors are refused, never
    computed on the host."""
    import torch
    from linear_recurrent_token_amd import autograd as A
    q = torch.zeros((1, 4, 1, 16))
    la = torch.zeros((1, 4, 1))
    with pytest.raises(ValueError):
        A.gated_delta_net(q, q, q, la, la)
    with pytest.raises(ValueError):
        A.short_conv(torch.zeros((1, 4, 8)), torch.zeros((8, 4)))
