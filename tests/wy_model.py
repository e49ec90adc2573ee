"""fp64 numpy model of the chunked (WY / generalised-Householder) form.

Test-only.  It is NOT the oracle: it writes out, step by step, the chunked
algebra the HIP kernels implement, so that a test can show the algebra equals
the token loop of the oracle (the ainew page, "DeltaNet (Parallelizing linear
transformers with delta rule)", states that each chunk's outputs follow from
the previous chunk's final state plus the chunk's own q, k, v, via a
reparameterisation whose printed form is cut off; the form below is derived
from the recurrence itself).

Per chunk with rows 1..C, state S entering the chunk:
  delta_r = beta_r (v_r - k_r S_{r-1}),   S_r = S + sum_{i<=r} k_i^T delta_i
  => (I + A) Delta = diag(beta) (V - K S),   A = tril(diag(beta) K K^T, -1)
  => Delta = T (V - K S),   T = (I + A)^{-1} diag(beta)   (lower triangular)
     O = Q S + tril(Q K^T) Delta   (diagonal included)
     S' = S + K^T Delta
A ragged last chunk is padded with k = 0, beta = 0 rows, which are exact
no-ops.
"""

from __future__ import annotations

import numpy as np


def wy_T(K, beta):
    """T = (I + tril(diag(beta) K K^T, -1))^{-1} diag(beta) by forward
    substitution, row by row: T[r] = beta_r e_r - sum_{i<r} A[r,i] T[i]."""
    C = K.shape[0]
    A = np.tril(beta[:, None] * (K @ K.T), -1)
    T = np.zeros((C, C))
    for r in range(C):
        T[r] = -A[r, :r] @ T[:r]
        T[r, r] = beta[r]
    return T


def chunked_forward(q, k, v, beta, S0, C):
    """Chunked forward for one head: q,k [L,dk], v [L,dv], beta [L], S0 [dk,dv]."""
    L, dk = k.shape
    dv = v.shape[1]
    n = -(-L // C)
    pad = n * C - L
    if pad:
        q = np.concatenate([q, np.zeros((pad, dk))])
        k = np.concatenate([k, np.zeros((pad, dk))])
        v = np.concatenate([v, np.zeros((pad, dv))])
        beta = np.concatenate([beta, np.zeros(pad)])
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    o = np.zeros((n * C, dv))
    for c in range(n):
        sl = slice(c * C, (c + 1) * C)
        Kc, Qc, Vc, bc = k[sl], q[sl], v[sl], beta[sl]
        T = wy_T(Kc, bc)
        D = T @ (Vc - Kc @ S)
        o[sl] = Qc @ S + np.tril(Qc @ Kc.T) @ D
        S = S + Kc.T @ D
    return o[:L], S


def chunked_forward_wu(q, k, v, beta, S0, C):
    """Same, in the W/U form: W = T K, U = T V, Delta = U - W S."""
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    o = np.zeros((L, dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        Kc, Qc, Vc, bc = k[sl], q[sl], v[sl], beta[sl]
        T = wy_T(Kc, bc)
        W, U = T @ Kc, T @ Vc
        D = U - W @ S
        o[sl] = Qc @ S + np.tril(Qc @ Kc.T) @ D
        S = S + Kc.T @ D
    return o, S


# ---- gated (Gated DeltaNet) chunked form --------------------------------------
#
# Decay first, then the delta write on the decayed state.  Within a chunk, with
# g_r = log(alpha_1) + ... + log(alpha_r) (local rows 1..C, g_0 = 0) and the
# entering state S:
#   S_r = e^{g_r} S + sum_{i<=r} e^{g_r - g_i} k_i^T delta_i
#   delta_r = beta_r (v_r - e^{g_r} k_r S - sum_{i<r} e^{g_r - g_i} (k_r . k_i) delta_i)
#   => (I + A) Delta = diag(beta) (V - diag(e^g) K S),  A_ri = beta_r e^{g_r - g_i} (k_r . k_i), i < r
#      O  = diag(e^g) Q S + (tril(Q K^T) * e^{g_r - g_i}) Delta
#      S' = e^{g_C} S + K^T diag(e^{g_C - g}) Delta
# Every exponent is <= 0.  A zero alpha is floored at LOG_FLOOR (its factor
# e^{-87.3} ~ 1e-38 stands for 0, as in the kernels); padded rows have
# alpha = 1, k = 0, beta = 0 (exact no-ops).  With sub-blocks of SB rows the
# state and outputs are regrouped as the matrix-core scan does:
#   S_{b+1} = e^{G_{b+1} - G_b} S_b + sum_{i in b} e^{G_{b+1} - g_i} k_i^T delta_i,
#   O_b     = diag(e^{g - G_b}) Q_b S_b + (tril(Q_b K_b^T) * e^{g_r - g_i}) Delta_b,
# with G_b the g of the last row before sub-block b (G_0 = 0).

LOG_FLOOR = float(np.log(np.float32(1.1754944e-38)))


def gated_chunked_forward(q, k, v, alpha, beta, S0, C, SB=None):
    L, dk = k.shape
    dv = v.shape[1]
    n = -(-L // C)
    pad = n * C - L
    if pad:
        q = np.concatenate([q, np.zeros((pad, dk))])
        k = np.concatenate([k, np.zeros((pad, dk))])
        v = np.concatenate([v, np.zeros((pad, dv))])
        beta = np.concatenate([beta, np.zeros(pad)])
        alpha = np.concatenate([alpha, np.ones(pad)])
    la = np.maximum(np.log(np.maximum(alpha, 0.0) + 0.0, where=alpha > 0,
                           out=np.full(alpha.shape, -np.inf)), LOG_FLOOR)
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    o = np.zeros((n * C, dv))
    for c in range(n):
        sl = slice(c * C, (c + 1) * C)
        Kc, Qc, Vc, bc = k[sl], q[sl], v[sl], beta[sl]
        g = np.cumsum(la[sl])
        E = np.exp(np.minimum(g[:, None] - g[None, :], 0.0))   # e^{g_r - g_i}, used for i <= r
        A = np.tril(bc[:, None] * E * (Kc @ Kc.T), -1)
        T = np.linalg.solve(np.eye(C) + A, np.diag(bc))
        D = T @ (Vc - np.exp(g)[:, None] * (Kc @ S))
        if SB is None:
            o[sl] = np.exp(g)[:, None] * (Qc @ S) + (np.tril(Qc @ Kc.T) * E) @ D
            S = np.exp(g[-1]) * S + Kc.T @ (np.exp(g[-1] - g)[:, None] * D)
        else:
            Sb, Gb = S, 0.0
            for b0 in range(0, C, SB):
                bs = slice(b0, b0 + SB)
                gb = g[bs]
                Eb = E[bs, bs]
                o[c * C + b0:c * C + b0 + SB] = (np.exp(gb - Gb)[:, None] * (Qc[bs] @ Sb)
                                                 + (np.tril(Qc[bs] @ Kc[bs].T) * Eb) @ D[bs])
                Gn = gb[-1]
                Sb = np.exp(Gn - Gb) * Sb + Kc[bs].T @ (np.exp(Gn - gb)[:, None] * D[bs])
                Gb = Gn
            S = Sb
    return o[:L], S


def chunked_backward(q, k, v, beta, S0, dO, dS_final, C):
    """fp64 model of the chunked backward the HIP kernels implement, per
    chunk with entering state S and exit gradient G' = dL/dS':
        forward:  X = (I + A)^{-1}, A = tril(diag(beta) K K^T, -1),
                  T = X diag(beta), R = V - K S, Delta = T R,
                  M = tril(Q K^T) (diagonal included),
                  O = Q S + M Delta, S' = S + K^T Delta
        backward: dDelta = M^T dO + K G',  dR = T^T dDelta,  dV = dR,
                  dS = G' + Q^T dO - K^T dR,
                  dM = tril(dO Delta^T),  dQ = dO S^T + dM K,
                  dT = dDelta R^T,  dX = dT diag(beta),
                  dbeta_i += sum_r X_ri dT_ri,
                  dA = -X^T dX X^T (strictly lower part),
                  W = diag(beta) dA,  dbeta_r += sum_i dA_ri (k_r . k_i),
                  dK = dM^T Q + Delta G'^T - dR S^T + W K + W^T K.
    Returns (dq, dk, dv, dbeta, dS0)."""
    q, k, v, beta, dO = (np.asarray(x, np.float64) for x in (q, k, v, beta, dO))
    B, H, L, dk_ = k.shape
    dv_ = v.shape[-1]
    outs = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(beta),
            np.zeros((B, H, dk_, dv_))]
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk_, dv_)) if S0 is None else np.asarray(S0, np.float64)[b, h].copy()
            saved = []
            for t0 in range(0, L, C):
                sl = slice(t0, min(t0 + C, L))
                K, V, bt = k[b, h, sl], v[b, h, sl], beta[b, h, sl]
                A = np.tril(bt[:, None] * (K @ K.T), -1)
                X = np.linalg.inv(np.eye(len(bt)) + A)
                T = X * bt[None, :]
                R = V - K @ S
                D = T @ R
                saved.append((sl, S.copy(), X, T, R, D))
                S = S + K.T @ D
            G = np.zeros((dk_, dv_)) if dS_final is None else np.asarray(dS_final, np.float64)[b, h].copy()
            for sl, S, X, T, R, D in reversed(saved):
                Q, K, bt, dOc = q[b, h, sl], k[b, h, sl], beta[b, h, sl], dO[b, h, sl]
                M = np.tril(Q @ K.T)
                dD = M.T @ dOc + K @ G
                dR = T.T @ dD
                dM = np.tril(dOc @ D.T)
                dT = dD @ R.T
                dX = dT * bt[None, :]
                db = np.sum(X * dT, axis=0)
                dA = np.tril(-X.T @ dX @ X.T, -1)
                W = bt[:, None] * dA
                db = db + np.sum(dA * (K @ K.T), axis=1)
                outs[0][b, h, sl] = dOc @ S.T + dM @ K
                outs[1][b, h, sl] = dM.T @ Q + D @ G.T - dR @ S.T + W @ K + W.T @ K
                outs[2][b, h, sl] = dR
                outs[3][b, h, sl] = db
                G = G + Q.T @ dOc - K.T @ dR
            outs[4][b, h] = G
    return tuple(outs)
