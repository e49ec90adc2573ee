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
