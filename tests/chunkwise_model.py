"""Test-only fp64 model of the chunkwise (UT / WY) algebra the HIP kernels use
for the Gated DeltaNet branch.  It is NOT the oracle: the tests check it
against the oracle's per-token recurrence, which validates the algebra the
kernels implement before any GPU run.

Per chunk of C tokens starting from state S0 (key-major, [Dk, Dv]):
  g_r   = sum_{i<=r} log alpha_i        (gamma_r = exp(g_r))
  A     = strict_tril(exp(g_r - g_i) * k_r . k_i)
  T     = (I + diag(beta) A)^-1          (unit lower triangular)
  W     = T diag(beta * gamma) K ;  U~ = T diag(beta) V
  U     = U~ - W S0                      (the per-token delta-rule "errors")
  P     = tril(exp(g_r - g_i) * q_r . k_i)   (diagonal included)
  O     = diag(gamma) Q S0 + P U
  S_end = gamma_C S0 + K~^T U,  K~ = diag(exp(g_C - g_i)) K
The state is committed (S0 <- S_end) only for linear-routed chunks.
"""
import numpy as np


def gdn_chunkwise(q, k, v, alpha, beta, route_bgc, S_init=None, chunk=64):
    q, k, v, alpha, beta = (np.asarray(a, np.float64) for a in (q, k, v, alpha, beta))
    B, H, L, Dk = q.shape
    Dv = v.shape[3]
    G = route_bgc.shape[1]
    o = np.zeros((B, H, L, Dv))
    S_fin = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            r = route_bgc[b, h // (H // G)]
            S = np.zeros((Dk, Dv)) if S_init is None else np.asarray(S_init, np.float64)[b, h].copy()
            for c0 in range(0, L, chunk):
                sl = slice(c0, c0 + chunk)
                Q, K, V = q[b, h, sl], k[b, h, sl], v[b, h, sl]
                a, be = alpha[b, h, sl], beta[b, h, sl]
                C = len(a)
                g = np.cumsum(np.log(a))
                gam = np.exp(g)
                Gm = np.exp(g[:, None] - g[None, :])
                A = np.tril(Gm * (K @ K.T), -1)
                T = np.linalg.inv(np.eye(C) + be[:, None] * A)
                W = T @ ((be * gam)[:, None] * K)
                Ut = T @ (be[:, None] * V)
                U = Ut - W @ S
                P = np.tril(Gm * (Q @ K.T))
                o[b, h, sl] = gam[:, None] * (Q @ S) + P @ U
                if C == chunk and r[c0 // chunk] == 1:
                    Kt = np.exp(g[-1] - g)[:, None] * K
                    S = gam[-1] * S + Kt.T @ U
            S_fin[b, h] = S
    return o, S_fin


def gdn_chunkwise_backward(q, k, v, alpha, beta, route_bgc, d_o, S_init=None, dS_final=None, chunk=64):
    """Test-only fp64 model of the chunkwise gradient the HIP kernels use
    (the derivative of the chunk form above, chunk by chunk in reverse).

    With Gc = d loss / d carried state after chunk c (dS_final after the last)
    and S0 the chunk's start state; dSe = Gc for a linear-routed chunk (its end
    state is committed), 0 otherwise:
      dU  = P^T dO + K~ dSe
      dS0 = gamma_C dSe + Q^T diag(gamma) dO - W^T dU  (+ Gc if not committed)
      dgate = <Gc, (gamma_C - 1) S0 + K~^T U>
    and inside the chunk, with Bv = diag(b) V, Bk = diag(b gamma) K:
      dP = tril(dO U^T),  dK~ = U dSe^T,  dQ = diag(gamma) dO S0^T + F K
      dW = -dU S0^T,  dT = dU Bv^T + dW Bk^T,  dM = -T^T dT T^T
      dV = diag(b) T^T dU,  dK = diag(b gamma) T^T dW + E K + E^T K + F^T Q
           + diag(exp(g_C - g)) dK~
      E = beta * strict_tril(dM) * exp(g_r - g_i),  F = dP * exp(g_r - g_i)
      dbeta = rowsum(V * T^T dU) + gamma rowsum(K * T^T dW) + rowsum(dM_sl * A)
      dg (log-decay) from gamma, A, P and K~, reverse-cumsummed into
      d log alpha, then dalpha = d log alpha / alpha (alpha > 0).
    Returns dq, dk, dv, dalpha, dbeta, dS_init, dgate."""
    q, k, v, alpha, beta, d_o = (np.asarray(a, np.float64) for a in (q, k, v, alpha, beta, d_o))
    B, H, L, Dk = q.shape
    Dv = v.shape[3]
    G_ = route_bgc.shape[1]
    nc = L // chunk
    assert nc * chunk == L
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dalpha, dbeta = np.zeros_like(alpha), np.zeros_like(beta)
    dS_init = np.zeros((B, H, Dk, Dv))
    dgate = np.zeros((B, H, nc))
    for b in range(B):
        for h in range(H):
            r = route_bgc[b, h // (H // G_)]
            S = np.zeros((Dk, Dv)) if S_init is None else np.asarray(S_init, np.float64)[b, h].copy()
            starts = []
            for c in range(nc):
                starts.append(S.copy())
                sl = slice(c * chunk, (c + 1) * chunk)
                if r[c] == 1:
                    Q, K, V = q[b, h, sl], k[b, h, sl], v[b, h, sl]
                    a, be = alpha[b, h, sl], beta[b, h, sl]
                    g = np.cumsum(np.log(a))
                    gam = np.exp(g)
                    A = np.tril(np.exp(g[:, None] - g[None, :]) * (K @ K.T), -1)
                    T = np.linalg.inv(np.eye(chunk) + be[:, None] * A)
                    U = T @ (be[:, None] * V) - T @ ((be * gam)[:, None] * K) @ S
                    S = gam[-1] * S + (np.exp(g[-1] - g)[:, None] * K).T @ U
            Gc = np.zeros((Dk, Dv)) if dS_final is None else np.asarray(dS_final, np.float64)[b, h].copy()
            for c in reversed(range(nc)):
                sl = slice(c * chunk, (c + 1) * chunk)
                S0 = starts[c]
                Q, K, V, dO = q[b, h, sl], k[b, h, sl], v[b, h, sl], d_o[b, h, sl]
                a, be = alpha[b, h, sl], beta[b, h, sl]
                lin = r[c] == 1
                g = np.cumsum(np.log(a))
                gam = np.exp(g)
                Gm = np.exp(g[:, None] - g[None, :])
                A = np.tril(Gm * (K @ K.T), -1)
                T = np.linalg.inv(np.eye(chunk) + be[:, None] * A)
                Bv = be[:, None] * V
                Bk = (be * gam)[:, None] * K
                W = T @ Bk
                U = T @ Bv - W @ S0
                P = np.tril(Gm * (Q @ K.T))
                ec = np.exp(g[-1] - g)
                Kt = ec[:, None] * K
                dSe = Gc if lin else np.zeros_like(Gc)
                dgate[b, h, c] = np.sum(Gc * ((gam[-1] - 1.0) * S0 + Kt.T @ U))
                dU = P.T @ dO + Kt @ dSe
                dS0 = gam[-1] * dSe + Q.T @ (gam[:, None] * dO) - W.T @ dU + (0.0 if lin else Gc)
                dP = np.tril(dO @ U.T)
                dKt = U @ dSe.T
                dOS = dO @ S0.T
                dQ = gam[:, None] * dOS
                dgam = np.sum(Q * dOS, axis=1)
                dW = -dU @ S0.T
                dT = dU @ Bv.T + dW @ Bk.T
                TdU, TdW = T.T @ dU, T.T @ dW
                dV = be[:, None] * TdU
                dK = (be * gam)[:, None] * TdW
                dbe = np.sum(V * TdU, axis=1) + gam * np.sum(K * TdW, axis=1)
                dgam += be * np.sum(K * TdW, axis=1)
                dM = np.tril(-T.T @ dT @ T.T, -1)
                dbe += np.sum(dM * A, axis=1)
                dA = be[:, None] * dM
                E = dA * Gm
                dK += E @ K + E.T @ K
                dg = np.sum(dA * A, axis=1) - np.sum(dA * A, axis=0)
                F = dP * Gm
                dQ += F @ K
                dK += F.T @ Q
                dg += np.sum(dP * P, axis=1) - np.sum(dP * P, axis=0)
                dK += ec[:, None] * dKt
                ts = np.sum(Kt * dKt, axis=1)
                dg -= ts
                dg += gam * dgam
                dg[-1] += ts.sum() + gam[-1] * np.sum(dSe * S0)
                dla = np.cumsum(dg[::-1])[::-1]
                dq[b, h, sl], dk[b, h, sl], dv[b, h, sl] = dQ, dK, dV
                dalpha[b, h, sl] = dla / a
                dbeta[b, h, sl] = dbe
                Gc = dS0
            dS_init[b, h] = Gc
    return dq, dk, dv, dalpha, dbeta, dS_init, dgate
