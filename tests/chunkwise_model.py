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
