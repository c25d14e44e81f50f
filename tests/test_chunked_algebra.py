"""The chunkwise (WY/UT) rewrite the GPU kernels use equals the sequential
oracle to rounding, including chunk size 1 (where it degenerates to the
recurrence itself), ragged tail chunks and T shorter than one chunk."""
import numpy as np
import pytest

import oracle
from tests import chunked_ref as cr


def _inp(seed, T, d, kda=False, variant="gdn"):
    r = np.random.default_rng(seed)
    B, H = 1, 2
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, d))
    beta = r.uniform(0.05, 0.95, (B, T, H))
    la = -r.uniform(0.0, 0.8, (B, T, H, d) if kda else (B, T, H))
    h0 = r.standard_normal((B, H, d, d))
    do = r.standard_normal((B, T, H, d))
    dht = r.standard_normal((B, H, d, d))
    return q, k, v, la, beta, h0, do, dht


@pytest.mark.parametrize("variant", ["gdn", "ssd", "kda"])
@pytest.mark.parametrize("C", [1, 2, 4, 16])
@pytest.mark.parametrize("T", [1, 7, 64, 61])
@pytest.mark.parametrize("d", [4, 8])
def test_chunked_forward_equals_sequential(variant, C, T, d):
    q, k, v, la, beta, h0, _, _ = _inp(T * 31 + C * 7 + d, T, d, kda=variant == "kda")
    o, ht = oracle.fwd(variant, q, k, v, la, beta, h0)
    oc, hc = cr.fwd(variant, q, k, v, la, beta, h0, C)
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12 * max(1, np.abs(o).max()))
    np.testing.assert_allclose(hc, ht, rtol=0, atol=1e-12 * max(1, np.abs(ht).max()))


@pytest.mark.parametrize("C", [1, 4, 16])
@pytest.mark.parametrize("T", [1, 7, 61])
def test_chunked_gdn_backward_equals_bptt(C, T):
    q, k, v, la, beta, h0, do, dht = _inp(T * 13 + C, T, 4)
    ref = oracle.bwd("gdn", q, k, v, la, beta, h0, do, dht)
    got = cr.gdn_bwd(q, k, v, la, beta, h0, do, dht, C)
    for name, a, b in zip(["dq", "dk", "dv", "dlog_a", "dbeta", "dh0"], got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1, np.abs(b).max()), err_msg=name)


@pytest.mark.parametrize("C", [1, 4, 16])
@pytest.mark.parametrize("T", [1, 7, 61])
def test_chunked_kda_backward_equals_bptt(C, T):
    """The effective-operand chunk backward of KDA (per-dimension gates)
    equals back-propagation through the sequential recurrence."""
    q, k, v, la, beta, h0, do, dht = _inp(T * 17 + C, T, 4, kda=True)
    ref = oracle.bwd("kda", q, k, v, la, beta, h0, do, dht)
    got = cr.kda_bwd(q, k, v, la, beta, h0, do, dht, C)
    for name, a, b in zip(["dq", "dk", "dv", "dlog_a", "dbeta", "dh0"], got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1, np.abs(b).max()), err_msg=name)
