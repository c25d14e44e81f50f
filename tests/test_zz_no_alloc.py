"""gdn_fwd_noalloc (the Gated DeltaNet forward with the library's static
per-GPU workspace, for callers that cannot allocate) against gdn_fwd with a
caller workspace, through the C ABI: two calls in a row, the second smaller
(the array keeps the first call's contents), and the size limit."""
import ctypes
import sys

import pytest
import torch

from linear_recurrent_token_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_gdn_fwd_twice():
    import linear_recurrent_token_amd as L
    lib = L.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [
        # B, T, H, d_k, d_v, chunk, dtype, gate_shift, h0_std
        (2, 300, 4, 128, 128, 64, torch.bfloat16, -2.0, 0.1),
        (1, 77, 2, 64, 32, 16, torch.float32, -6.0, 0.1),  # smaller: stale contents of the first call
    ]
    for B, T, H, dk, dv, chunk, dt, shift, h0s in cases:
        say(f"[noalloc] B={B} T={T} H={H} dk={dk} dv={dv} chunk={chunk} {dt}")
        inp = synth.make_inputs("gdn_fwd", B, T, H, dk, dv, dtype=dt, seed=7, device="cuda", gate_shift=shift,
                                h0_std=h0s)
        q, k, v, la, beta, h0 = (inp[n] for n in ("q", "k", "v", "log_a", "beta", "h0"))
        ref_o, ref_ht = L.gdn_fwd(q, k, v, la, beta, h0, chunk=chunk)
        o = torch.full_like(ref_o, float("nan"))
        ht = torch.full_like(ref_ht, float("nan"))
        code = L.LRT_BF16 if dt == torch.bfloat16 else L.LRT_F32
        rc = lib.gdn_fwd_noalloc(_p(q), _p(k), _p(v), _p(la), _p(beta), _p(h0), _p(o), _p(ht), B, T, H, dk, dv,
                                 chunk, code, stream)
        assert rc == 0, L.status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(ht, ref_ht)
        # the Python binding of the same entry point
        o2, ht2 = L.gdn_fwd_noalloc(q, k, v, la, beta, h0, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(ht2, ref_ht)


def test_noalloc_rejects_sizes_beyond_the_array():
    import linear_recurrent_token_amd as L
    lib = L.lib()
    B, T, H, dk, dv, chunk = 16, 2048, 8, 128, 128, 64
    need = L.workspace_bytes(L.OP_GDN_FWD, B, T, H, dk, dv, chunk, L.LRT_BF16)
    assert need > L.NOALLOC_MAX_BYTES
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: the size check comes first
    rc = lib.gdn_fwd_noalloc(fake, fake, fake, fake, fake, None, fake, None, B, T, H, dk, dv, chunk, L.LRT_BF16, None)
    assert rc == -9 and "LRT_NOALLOC_MAX_BYTES" in L.status_string(rc)
