"""fp64 numpy statement of the chunkwise (WY / UT) form of the mixers.

Test infrastructure: the tests use it to show that the chunked algebra the
GPU kernels implement is an exact rewrite of the sequential recurrence (it
must equal the oracle to rounding), and to inspect per-chunk intermediates.
It is not the oracle and the oracle does not use it.

Derivation (state H = S^T, [d_k, d_v]; chunk rows i, j; Hn = state at the
chunk start; g = within-chunk inclusive cumsum of log a):
  u_i = b_i (v_i - a_i H_{i-1}^T k_i) unrolled inside the chunk gives
  (I + A) U = diag(b) V - diag(b gamma) K Hn  with
  A_ij = b_i (k_i . k_j) exp(g_i - g_j)  for j < i,   gamma_i = exp(g_i).
  Hence U = U' - W Hn,  W = T diag(b gamma) K,  U' = T diag(b) V,  T = (I+A)^-1,
  O = diag(gamma) Q Hn + ((Q K^T) o Gamma) U   (Gamma_ij = exp(g_i - g_j), j <= i),
  H_next = gamma_C Hn + Ktil^T U,  Ktil_j = exp(g_C - g_j) k_j.
KDA replaces the scalar g by a per-key-dimension G (C x d_k).
"""
import numpy as np


def _chunks(T, C):
    return [(s, min(T, s + C)) for s in range(0, T, C)]


def fwd(variant, q, k, v, la, beta, h0, C):
    q, k, v, la = (np.asarray(x, np.float64) for x in (q, k, v, la))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ht = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            Hn = np.zeros((dk, dv)) if h0 is None else np.asarray(h0, np.float64)[b, h].copy()
            for s, e in _chunks(T, C):
                Q, K, V = q[b, s:e, h], k[b, s:e, h], v[b, s:e, h]
                n = e - s
                if variant == "kda":
                    G = np.cumsum(la[b, s:e, h], axis=0)                 # [n, dk]
                    E = np.exp(G[:, None, :] - G[None, :, :])            # [i, j, d]
                    mask = np.tril(np.ones((n, n)))
                    Aqk = np.einsum("id,jd,ijd->ij", Q, K, E) * mask
                    bt = np.asarray(beta, np.float64)[b, s:e, h]
                    A = bt[:, None] * np.einsum("id,jd,ijd->ij", K, K, E) * np.tril(np.ones((n, n)), -1)
                    Tm = np.linalg.inv(np.eye(n) + A)
                    W = Tm @ (bt[:, None] * K * np.exp(G))
                    U = Tm @ (bt[:, None] * V) - W @ Hn
                    o[b, s:e, h] = (Q * np.exp(G)) @ Hn + Aqk @ U
                    Hn = np.exp(G[-1])[:, None] * Hn + (K * np.exp(G[-1][None, :] - G)).T @ U
                    continue
                g = np.cumsum(la[b, s:e, h])
                gam = np.exp(g)
                Gam = np.tril(np.exp(g[:, None] - g[None, :]))
                if variant == "ssd":
                    U = V
                else:
                    bt = np.asarray(beta, np.float64)[b, s:e, h]
                    A = np.tril(bt[:, None] * (K @ K.T) * Gam, -1)
                    Tm = np.linalg.inv(np.eye(n) + A)
                    W = Tm @ ((bt * gam)[:, None] * K)
                    U = Tm @ (bt[:, None] * V) - W @ Hn
                o[b, s:e, h] = gam[:, None] * (Q @ Hn) + ((Q @ K.T) * Gam) @ U
                Hn = gam[-1] * Hn + (np.exp(g[-1] - g)[:, None] * K).T @ U
            ht[b, h] = Hn
    return o, ht


def gdn_bwd(q, k, v, la, beta, h0, do, dht, C):
    """Chunked backward of GDN; returns (dq, dk, dv, dlog_a, dbeta, dh0)."""
    q, k, v, la, beta, do = (np.asarray(x, np.float64) for x in (q, k, v, la, beta, do))
    B, T, H, dk = q.shape
    dv_ = v.shape[-1]
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(la),
           np.zeros_like(beta), np.zeros((B, H, dk, dv_))]
    for b in range(B):
        for h in range(H):
            Hn = np.zeros((dk, dv_)) if h0 is None else np.asarray(h0, np.float64)[b, h].copy()
            states = []
            for s, e in _chunks(T, C):
                states.append(Hn.copy())
                _, Hn = _gdn_chunk(q[b, s:e, h], k[b, s:e, h], v[b, s:e, h], la[b, s:e, h],
                                   beta[b, s:e, h], Hn)
            dH = np.zeros((dk, dv_)) if dht is None else np.asarray(dht, np.float64)[b, h].copy()
            for ci in reversed(range(len(states))):
                s, e = _chunks(T, C)[ci]
                Hn = states[ci]
                Q, K, V, dO = q[b, s:e, h], k[b, s:e, h], v[b, s:e, h], do[b, s:e, h]
                bt = beta[b, s:e, h]
                g = np.cumsum(la[b, s:e, h])
                n = e - s
                gam = np.exp(g)
                Gam = np.tril(np.exp(g[:, None] - g[None, :]))
                KK = K @ K.T
                A = np.tril(bt[:, None] * KK * Gam, -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                X = (bt * gam)[:, None] * K
                Y = bt[:, None] * V
                W = Tm @ X
                U = Tm @ Y - W @ Hn
                P = (Q @ K.T) * Gam
                kt = np.exp(g[-1] - g)
                Kt = kt[:, None] * K
                dU = P.T @ dO + Kt @ dH
                dHn = gam[-1] * dH + Q.T @ (gam[:, None] * dO) - W.T @ dU
                dS = (dO @ U.T) * Gam                         # gradient of Q K^T (masked)
                dQ = gam[:, None] * (dO @ Hn.T) + dS @ K
                dK = dS.T @ Q
                dKt = U @ dH.T
                dK += kt[:, None] * dKt
                dW = -dU @ Hn.T
                dT = dW @ X.T + dU @ Y.T
                dX = Tm.T @ dW
                dY = Tm.T @ dU
                dV = bt[:, None] * dY
                cx = np.sum(dX * K, 1)
                dbt = np.sum(dY * V, 1) + gam * cx
                dK += (bt * gam)[:, None] * dX
                dA = np.tril(-(Tm.T @ dT @ Tm.T), -1)
                M = dA * bt[:, None] * Gam
                dbt += np.sum(dA * Gam * KK, 1)
                dK += M @ K + M.T @ K
                EP = dS * (Q @ K.T)                          # dGamma o Gamma from P
                EA = dA * A
                sj = np.sum(dKt * Kt, 1)
                dg = gam * np.sum(dO * (Q @ Hn), 1)
                dg += EP.sum(1) - EP.sum(0) + EA.sum(1) - EA.sum(0)
                dg += bt * gam * cx
                dg -= sj
                dg[-1] += sj.sum() + gam[-1] * np.sum(dH * Hn)
                out[0][b, s:e, h] = dQ
                out[1][b, s:e, h] = dK
                out[2][b, s:e, h] = dV
                out[3][b, s:e, h] = np.cumsum(dg[::-1])[::-1]
                out[4][b, s:e, h] = dbt
                dH = dHn
            out[5][b, h] = dH
    return tuple(out)


def kda_bwd(q, k, v, la, beta, h0, do, dht, C):
    """Chunked backward of KDA; returns (dq, dk, dv, dlog_a, dbeta, dh0).

    Written in effective operands (G = within-chunk per-dimension cumsum,
    E = exp(G), E_C its last row):  Qh = Q o E,  Kh = K o E,  Kb = K o E^-1,
    Kt = K o (E_C / E).  The chunk is then the Gated DeltaNet chunk with
    Gamma = 1 and the one K split by use:
      A = strict_lower(diag(b) Kh Kb^T),  T = (I + A)^-1,  W = T diag(b) Kh,
      U = T diag(b) V - W Hn,  O = Qh Hn + lower(Qh Kb^T) U,
      H_next = diag(E_C) Hn + Kt^T U.
    The GDN chunk backward gives dQh, dKh, dKb, dKt and dE_C; then
      dQ = dQh o E,  dK = dKh o E + dKb o E^-1 + dKt o (E_C / E),
      dG_t = Qh o dQh + Kh o dKh - Kb o dKb - Kt o dKt   (row t),
      dG_C += sum_t Kt o dKt + E_C o dE_C,
    and d log a is the within-chunk reverse cumsum of dG, per dimension.
    """
    q, k, v, la, beta, do = (np.asarray(x, np.float64) for x in (q, k, v, la, beta, do))
    B, T, H, dk = q.shape
    dv_ = v.shape[-1]
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(la),
           np.zeros_like(beta), np.zeros((B, H, dk, dv_))]
    for b in range(B):
        for h in range(H):
            Hn = np.zeros((dk, dv_)) if h0 is None else np.asarray(h0, np.float64)[b, h].copy()
            chunks = _chunks(T, C)
            states = []
            for s, e in chunks:
                states.append(Hn.copy())
                _, Hn = _kda_chunk(q[b, s:e, h], k[b, s:e, h], v[b, s:e, h], la[b, s:e, h], beta[b, s:e, h], Hn)
            dH = np.zeros((dk, dv_)) if dht is None else np.asarray(dht, np.float64)[b, h].copy()
            for ci in reversed(range(len(chunks))):
                s, e = chunks[ci]
                Hn = states[ci]
                Q, K, V, dO = q[b, s:e, h], k[b, s:e, h], v[b, s:e, h], do[b, s:e, h]
                bt = beta[b, s:e, h]
                n = e - s
                G = np.cumsum(la[b, s:e, h], axis=0)
                E, EC = np.exp(G), np.exp(G[-1])
                Qh, Kh, Kb, Kt = Q * E, K * E, K / E, K * (EC[None, :] / E)
                A = np.tril(bt[:, None] * (Kh @ Kb.T), -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                X = bt[:, None] * Kh
                Y = bt[:, None] * V
                W = Tm @ X
                U = Tm @ Y - W @ Hn
                P = np.tril(Qh @ Kb.T)
                # the GDN chunk backward with Gamma = 1, per effective operand
                dU = P.T @ dO + Kt @ dH
                dHn = EC[:, None] * dH + Qh.T @ dO - W.T @ dU
                dP = np.tril(dO @ U.T)
                dQh = dO @ Hn.T + dP @ Kb
                dKb = dP.T @ Qh
                dKt = U @ dH.T
                dEC = np.sum(dH * Hn, 1)
                dW = -dU @ Hn.T
                dX = Tm.T @ dW
                dY = Tm.T @ dU
                dT = dW @ X.T + dU @ Y.T
                dA = np.tril(-(Tm.T @ dT @ Tm.T), -1)
                dKh = (bt[:, None] * dA) @ Kb + bt[:, None] * dX
                dKb += (bt[:, None] * dA).T @ Kh
                dbt = np.sum(dA * (Kh @ Kb.T), 1) + np.sum(dX * Kh, 1) + np.sum(dY * V, 1)
                dV = bt[:, None] * dY
                # back to K, Q and the per-dimension gate
                dQ = dQh * E
                dK = dKh * E + dKb / E + dKt * (EC[None, :] / E)
                dG = Qh * dQh + Kh * dKh - Kb * dKb - Kt * dKt
                dG[-1] += np.sum(Kt * dKt, 0) + EC * dEC
                out[0][b, s:e, h] = dQ
                out[1][b, s:e, h] = dK
                out[2][b, s:e, h] = dV
                out[3][b, s:e, h] = np.cumsum(dG[::-1], axis=0)[::-1]
                out[4][b, s:e, h] = dbt
                dH = dHn
            out[5][b, h] = dH
    return tuple(out)


def _kda_chunk(Q, K, V, la, bt, Hn):
    G = np.cumsum(la, axis=0)
    n = len(G)
    E, EC = np.exp(G), np.exp(G[-1])
    A = np.tril(bt[:, None] * ((K * E) @ (K / E).T), -1)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ (bt[:, None] * K * E)
    U = Tm @ (bt[:, None] * V) - W @ Hn
    O = (Q * E) @ Hn + np.tril((Q * E) @ (K / E).T) @ U
    return O, EC[:, None] * Hn + (K * (EC[None, :] / E)).T @ U


def _gdn_chunk(Q, K, V, la, bt, Hn):
    g = np.cumsum(la)
    n = len(g)
    gam = np.exp(g)
    Gam = np.tril(np.exp(g[:, None] - g[None, :]))
    A = np.tril(bt[:, None] * (K @ K.T) * Gam, -1)
    Tm = np.linalg.inv(np.eye(n) + A)
    W = Tm @ ((bt * gam)[:, None] * K)
    U = Tm @ (bt[:, None] * V) - W @ Hn
    O = gam[:, None] * (Q @ Hn) + ((Q @ K.T) * Gam) @ U
    return O, gam[-1] * Hn + (np.exp(g[-1] - g)[:, None] * K).T @ U
