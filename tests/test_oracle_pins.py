"""Pins of the fp64 CPU oracle against facts fixed by the mixers' definitions.

The mixers (AMD ROCm blog "Pretraining hybrid LLMs with Primus", section "How
hybrid models are defined in Primus", mixer list under Table 2): Mamba2 decays
its state by one scalar gate per head; Gated DeltaNet adds the delta rule,
replacing the value stored under the current key; Kimi Delta Attention gives
the gate one value per key dimension.  Written in the state orientation
S (d_v x d_k):  S_t = a_t S_{t-1}(I - b k k^T) + b v k^T,  o_t = S_t q_t.

None of these checks re-types the oracle's loop: each one uses a different
fact (a hand-worked example, a closed form, an invariant, an independent
matrix-product form, a special case, or finite differences) chosen so that a
dropped term, a sign, an index or a transposed operand in the oracle fails.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed):
    return np.random.default_rng(seed)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def inputs(seed, B=1, T=9, H=2, dk=4, dv=3, kda=False, h0=True, unit_keys=True):
    r = rnd(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    if unit_keys:
        k = unit(k)
    v = r.standard_normal((B, T, H, dv))
    beta = r.uniform(0.05, 0.95, (B, T, H))
    la = -r.uniform(0.01, 1.0, (B, T, H, dk) if kda else (B, T, H))
    hh = r.standard_normal((B, H, dk, dv)) if h0 else None
    return q, k, v, la, beta, hh


# ---------------------------------------------------------------- hand example
def test_gdn_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "gdn_hand_T2_d2.json")))
    i = g["inputs"]
    f = lambda x: np.array(x, np.float64)
    q, k, v = (f(i[n])[None, :, None, :] for n in ("q", "k", "v"))
    beta = f(i["beta"])[None, :, None]
    la = np.log(f(i["a"]))[None, :, None]
    h0 = f(i["h0"])[None, None]
    o, ht = oracle.fwd("gdn", q, k, v, la, beta, h0)
    tol = g["tolerance_abs"]
    np.testing.assert_allclose(o[0, :, 0], f(g["expected"]["o"]), atol=tol, rtol=0)
    np.testing.assert_allclose(ht[0, 0], f(g["expected"]["ht"]), atol=tol, rtol=0)


# ------------------------------------------------- independent matrix-product form
def _s_form(variant, q, k, v, la, beta, h0):
    """S (d_v x d_k) orientation, explicit matrix products, one (b, h)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if h0 is None else h0.T.copy()
    outs = []
    for t in range(T):
        kt = k[t][:, None]
        if variant == "kda":
            D = np.diag(np.exp(la[t]))
            S = S @ D @ (np.eye(dk) - beta[t] * kt @ kt.T) + beta[t] * v[t][:, None] @ kt.T
        elif variant == "gdn":
            S = np.exp(la[t]) * S @ (np.eye(dk) - beta[t] * kt @ kt.T) + beta[t] * v[t][:, None] @ kt.T
        else:
            S = np.exp(la[t]) * S + v[t][:, None] @ kt.T
        outs.append(S @ q[t])
    return np.array(outs), S.T


@pytest.mark.parametrize("variant", ["gdn", "ssd", "kda"])
def test_matches_matrix_product_form(variant):
    kda = variant == "kda"
    q, k, v, la, beta, h0 = inputs(1, T=11, dk=5, dv=3, kda=kda, unit_keys=False)
    o, ht = oracle.fwd(variant, q, k, v, la, beta, h0)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            eo, eh = _s_form(variant, q[b, :, h], k[b, :, h], v[b, :, h], la[b, :, h],
                             beta[b, :, h], h0[b, h])
            np.testing.assert_allclose(o[b, :, h], eo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ht[b, h], eh, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ GDN pins
def test_gdn_beta_zero_is_pure_decay():
    q, k, v, la, beta, h0 = inputs(2, T=13)
    beta[:] = 0.0
    o, ht = oracle.fwd("gdn", q, k, v, la, beta, h0)
    cum = np.cumsum(la, axis=1)  # [B,T,H]
    exp_ht = np.exp(cum[:, -1])[:, :, None, None] * h0
    np.testing.assert_allclose(ht, exp_ht, rtol=1e-14, atol=0)
    exp_o = np.exp(cum)[..., None] * np.einsum("bhkv,bthk->bthv", h0, q)
    np.testing.assert_allclose(o, exp_o, rtol=1e-13, atol=1e-15)


def _orthonormal(r, n, d):
    m, _ = np.linalg.qr(r.standard_normal((d, d)))
    return m[:n]


def test_gdn_exact_retrieval_orthonormal_keys_any_h0():
    r = rnd(3)
    T, dk, dv = 6, 8, 5
    keys = _orthonormal(r, T, dk)
    k = keys[None, :, None, :]
    v = r.standard_normal((1, T, 1, dv))
    la = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    h0 = r.standard_normal((1, 1, dk, dv))
    # query at step t asks for the key written at step j(t) <= t
    js = [0, 0, 2, 1, 4, 3]
    q = keys[js][None, :, None, :]
    o, ht = oracle.fwd("gdn", q, k, v, la, beta, h0)
    for t, j in enumerate(js):
        np.testing.assert_allclose(o[0, t, 0], v[0, j, 0], rtol=0, atol=1e-13)
    for j in range(T):
        np.testing.assert_allclose(ht[0, 0].T @ keys[j], v[0, j, 0], rtol=0, atol=1e-13)


def test_gdn_per_step_delta_identity():
    # with |k_t| = 1:  H_t^T k_t = (1 - b_t) a_t H_{t-1}^T k_t + b_t v_t
    q, k, v, la, beta, h0 = inputs(4, T=10, B=2)
    for t in range(1, 10):
        _, hp = oracle.fwd("gdn", q[:, :t], k[:, :t], v[:, :t], la[:, :t], beta[:, :t], h0)
        _, hc = oracle.fwd("gdn", q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], la[:, :t + 1],
                           beta[:, :t + 1], h0)
        kt = k[:, t]  # [B,H,dk]
        lhs = np.einsum("bhkv,bhk->bhv", hc, kt)
        a, bt = np.exp(la[:, t])[..., None], beta[:, t][..., None]
        rhs = (1 - bt) * a * np.einsum("bhkv,bhk->bhv", hp, kt) + bt * v[:, t]
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)


@pytest.mark.parametrize("variant", ["gdn", "ssd", "kda"])
def test_joint_linearity_in_v_and_h0(variant):
    kda = variant == "kda"
    q, k, v1, la, beta, h1 = inputs(5, kda=kda)
    _, _, v2, _, _, h2 = inputs(6, kda=kda)
    al = 0.37
    o1, t1 = oracle.fwd(variant, q, k, v1, la, beta, h1)
    o2, t2 = oracle.fwd(variant, q, k, v2, la, beta, h2)
    o3, t3 = oracle.fwd(variant, q, k, al * v1 + v2, la, beta, al * h1 + h2)
    np.testing.assert_allclose(o3, al * o1 + o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(t3, al * t1 + t2, rtol=0, atol=1e-13)


def test_gdn_orthogonal_keys_equals_ssd_with_scaled_values():
    r = rnd(7)
    T, dk, dv = 7, 8, 4
    keys = _orthonormal(r, T, dk) * r.uniform(0.5, 2.0, (T, 1))  # orthogonal, not unit
    k = keys[None, :, None, :]
    q = r.standard_normal((1, T, 1, dk))
    v = r.standard_normal((1, T, 1, dv))
    la = -r.uniform(0.0, 1.0, (1, T, 1))
    beta = r.uniform(0.1, 0.9, (1, T, 1))
    o_g, t_g = oracle.fwd("gdn", q, k, v, la, beta, None)
    o_s, t_s = oracle.fwd("ssd", q, k, beta[..., None] * v, la, None, None)
    np.testing.assert_allclose(o_g, o_s, rtol=0, atol=1e-13)
    np.testing.assert_allclose(t_g, t_s, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ SSD pins
@pytest.mark.parametrize("T", [1, 17, 200])
def test_ssd_quadratic_closed_form(T):
    r = rnd(8 + T)
    B, H, dk, dv = 2, 2, 6, 5
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    la = -r.uniform(0.0, 0.3, (B, T, H))
    h0 = r.standard_normal((B, H, dk, dv))
    o, ht = oracle.fwd("ssd", q, k, v, la, None, h0)
    G = np.cumsum(la, axis=1)
    for b in range(B):
        for h in range(H):
            # o_t = sum_{s<=t} e^{G_t - G_s} (q_t . k_s) v_s + e^{G_t} h0^T q_t
            L = np.tril(np.exp(G[b, :, h][:, None] - G[b, :, h][None, :]))
            att = (q[b, :, h] @ k[b, :, h].T) * L
            exp = att @ v[b, :, h] + np.exp(G[b, :, h])[:, None] * (q[b, :, h] @ h0[b, h])
            np.testing.assert_allclose(o[b, :, h], exp, rtol=0, atol=1e-12)
            eh = np.exp(G[b, -1, h]) * h0[b, h] + (k[b, :, h] * np.exp(G[b, -1, h] - G[b, :, h])[:, None]).T @ v[b, :, h]
            np.testing.assert_allclose(ht[b, h], eh, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ KDA pins
def test_kda_uniform_gate_equals_gdn():
    q, k, v, la, beta, h0 = inputs(9, T=12)
    lak = np.repeat(la[..., None], q.shape[-1], axis=-1)
    o_g, t_g = oracle.fwd("gdn", q, k, v, la, beta, h0)
    o_k, t_k = oracle.fwd("kda", q, k, v, lak, beta, h0)
    np.testing.assert_allclose(o_k, o_g, rtol=0, atol=1e-13)
    np.testing.assert_allclose(t_k, t_g, rtol=0, atol=1e-13)


def test_kda_beta_zero_is_per_dim_decay():
    q, k, v, la, beta, h0 = inputs(10, T=9, kda=True)
    beta[:] = 0.0
    o, ht = oracle.fwd("kda", q, k, v, la, beta, h0)
    cum = np.cumsum(la, axis=1)  # [B,T,H,dk]
    np.testing.assert_allclose(ht, np.exp(cum[:, -1])[..., None] * h0, rtol=1e-14, atol=0)
    exp_o = np.einsum("bthk,bhkv->bthv", q * np.exp(cum), h0)
    np.testing.assert_allclose(o, exp_o, rtol=1e-13, atol=1e-15)


def test_kda_per_step_identity():
    # with |k_t| = 1:  H_t^T k_t = (1 - b_t) (Diag(a_t) H_{t-1})^T k_t + b_t v_t
    q, k, v, la, beta, h0 = inputs(11, T=8, kda=True)
    for t in range(1, 8):
        _, hp = oracle.fwd("kda", q[:, :t], k[:, :t], v[:, :t], la[:, :t], beta[:, :t], h0)
        _, hc = oracle.fwd("kda", q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], la[:, :t + 1],
                           beta[:, :t + 1], h0)
        kt = k[:, t]
        lhs = np.einsum("bhkv,bhk->bhv", hc, kt)
        X = np.exp(la[:, t])[..., None] * hp
        bt = beta[:, t][..., None]
        rhs = (1 - bt) * np.einsum("bhkv,bhk->bhv", X, kt) + bt * v[:, t]
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)


# ----------------------------------------------------- interface properties
@pytest.mark.parametrize("variant", ["gdn", "ssd", "kda"])
def test_state_chaining(variant):
    kda = variant == "kda"
    q, k, v, la, beta, h0 = inputs(12, T=21, kda=kda)
    o, ht = oracle.fwd(variant, q, k, v, la, beta, h0)
    t1 = 8
    oa, ha = oracle.fwd(variant, q[:, :t1], k[:, :t1], v[:, :t1], la[:, :t1], beta[:, :t1], h0)
    ob, hb = oracle.fwd(variant, q[:, t1:], k[:, t1:], v[:, t1:], la[:, t1:], beta[:, t1:], ha)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(hb, ht, rtol=0, atol=1e-13)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_column_range_equals_full(variant):
    kda = variant == "kda"
    q, k, v, la, beta, h0 = inputs(13, dv=7, kda=kda)
    o, ht = oracle.fwd(variant, q, k, v, la, beta, h0)
    o2, ht2 = oracle.fwd(variant, q, k, v, la, beta, h0, cols=(2, 3))
    np.testing.assert_array_equal(o2, o[..., 2:5])
    np.testing.assert_array_equal(ht2, ht[..., 2:5])


def test_typed_inputs_are_widened_exactly():
    import torch
    q, k, v, la, beta, h0 = inputs(14)
    qt, kt, vt = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    o_b, _ = oracle.fwd("gdn", qt, kt, vt, la, beta, h0)
    o_d, _ = oracle.fwd("gdn", qt.double(), kt.double(), vt.double(), la, beta, h0)
    np.testing.assert_array_equal(o_b, o_d)


# --------------------------------------------------------------- backward pins
def _loss(variant, q, k, v, la, beta, h0, do, dht):
    o, ht = oracle.fwd(variant, q, k, v, la, beta, h0)
    return float(np.sum(o * do) + np.sum(ht * dht))


@pytest.mark.parametrize("variant", ["gdn", "ssd", "kda"])
@pytest.mark.parametrize("T", [5, 13])
def test_backward_finite_differences(variant, T):
    kda = variant == "kda"
    r = rnd(20 + T)
    q, k, v, la, beta, h0 = inputs(21 + T, B=1, T=T, H=1, dk=4, dv=3, kda=kda, unit_keys=False)
    do = r.standard_normal((1, T, 1, 3))
    dht = r.standard_normal((1, 1, 4, 3))
    g = oracle.bwd(variant, q, k, v, la, beta, h0, do, dht)
    named = {"q": (q, g[0]), "k": (k, g[1]), "v": (v, g[2]), "log_a": (la, g[3]), "h0": (h0, g[5])}
    if variant != "ssd":
        named["beta"] = (beta, g[4])
    eps = 1e-6
    args = dict(q=q, k=k, v=v, log_a=la, beta=beta, h0=h0)
    for name, (x, gx) in named.items():
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = dict(args), dict(args)
            ap[name], am[name] = xp, xm
            lp = _loss(variant, ap["q"], ap["k"], ap["v"], ap["log_a"], ap["beta"], ap["h0"], do, dht)
            lm = _loss(variant, am["q"], am["k"], am["v"], am["log_a"], am["beta"], am["h0"], do, dht)
            fd[idx] = (lp - lm) / (2 * eps)
        scale = max(1.0, np.max(np.abs(fd)))
        assert np.max(np.abs(fd - gx)) <= 1e-6 * scale, (variant, name, np.max(np.abs(fd - gx)))


@pytest.mark.parametrize("variant", ["gdn", "ssd", "kda"])
def test_backward_linearity_identities(variant):
    kda = variant == "kda"
    r = rnd(30)
    q, k, v, la, beta, h0 = inputs(31, B=2, T=70, H=2, dk=5, dv=4, kda=kda)
    do = r.standard_normal(v.shape)
    dht = r.standard_normal(h0.shape)
    o, ht = oracle.fwd(variant, q, k, v, la, beta, h0)
    dq, dk, dv, dla, db, dh0 = oracle.bwd(variant, q, k, v, la, beta, h0, do, dht)
    # o is linear in q (ht does not depend on q)
    np.testing.assert_allclose(np.sum(dq * q), np.sum(do * o), rtol=1e-12)
    # o and ht are jointly linear in (v, h0)
    np.testing.assert_allclose(np.sum(dv * v) + np.sum(dh0 * h0), np.sum(do * o) + np.sum(dht * ht),
                               rtol=1e-12)


def test_gdn_backward_beta_zero_gives_zero_dv():
    r = rnd(32)
    q, k, v, la, beta, h0 = inputs(33, T=15)
    beta[:] = 0.0
    do = r.standard_normal(v.shape)
    _, _, dv, _, _, _ = oracle.bwd("gdn", q, k, v, la, beta, h0, do, None)
    assert np.all(dv == 0.0)


def test_backward_segment_checkpointing_boundary():
    # T spans several checkpoint segments with a ragged last one; compare with
    # the gradient of a two-call split (chaining) computed by finite pieces.
    r = rnd(34)
    q, k, v, la, beta, h0 = inputs(35, B=1, T=150, H=1, dk=3, dv=2)
    do = r.standard_normal(v.shape)
    dq, dk, dv, dla, db, dh0 = oracle.bwd("gdn", q, k, v, la, beta, h0, do, None)
    # gradient wrt the state passed between two halves equals dh0 of the second half
    t1 = 97
    _, hmid = oracle.fwd("gdn", q[:, :t1], k[:, :t1], v[:, :t1], la[:, :t1], beta[:, :t1], h0)
    g2 = oracle.bwd("gdn", q[:, t1:], k[:, t1:], v[:, t1:], la[:, t1:], beta[:, t1:], hmid,
                    do[:, t1:], None)
    g1 = oracle.bwd("gdn", q[:, :t1], k[:, :t1], v[:, :t1], la[:, :t1], beta[:, :t1], h0,
                    do[:, :t1], g2[5])
    np.testing.assert_allclose(np.concatenate([g1[0], g2[0]], 1), dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([g1[1], g2[1]], 1), dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([g1[3], g2[3]], 1), dla, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g1[5], dh0, rtol=0, atol=1e-12)
