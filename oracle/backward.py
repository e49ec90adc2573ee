"""fp64 CPU oracle for the gradient of the delta-rule forward (reverse mode).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path.

What it computes.  The pages call the chunked form a hardware-efficient way
to train in linear time (page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説",
section "DeltaNet (Parallelizing linear transformers with delta rule)") but
print no backward pass.  The gradient of the token loop (the same section;
``delta_rule_forward``) is fixed by calculus alone: with a loss whose
gradients with respect to the outputs are dO (``[B, H, L, d_v]``) and
dS_final (``[B, H, d_k, d_v]``), this function returns the gradients with
respect to q, k, v, beta and S0 by running the loop backwards.  Per token,
with S_{t-1} the state before token t and S_t after it:
    forward:  r_t = v_t - k_t S_{t-1},  u_t = beta_t r_t,
              S_t = S_{t-1} + k_t^T u_t,  o_t = q_t S_t
    backward (t = L .. 1, G = dL/dS_t, starting from dS_final):
              G    += q_t^T dO_t
              dq_t  = dO_t S_t^T
              du    = k_t G
              dv_t  = beta_t du
              dbeta_t = du . r_t
              dk_t  = u_t G^T - beta_t du S_{t-1}^T
              G    <- G - beta_t k_t^T du          (= dL/dS_{t-1})
    dS0 = G at the end.
The states S_t come from a plain forward pass kept in memory (L + 1 states
per head), so the sizes here are kept small.

Pins (tests/test_oracle_backward.py): central finite differences of the
(separately pinned) forward oracle for every input, a closed form at
beta = 0, and planted mistakes in a copy of the loop that each fail one.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def delta_rule_backward(q, k, v, beta, S0: Optional[np.ndarray], dO,
                        dS_final: Optional[np.ndarray] = None
                        ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dq, dk, dv, dbeta, dS0) of the delta-rule forward.

    q, k: ``[B, H, L, d_k]``; v, dO: ``[B, H, L, d_v]``; beta: ``[B, H, L]``;
    S0, dS_final: ``[B, H, d_k, d_v]`` or None (zero).  dS0 is returned
    whether or not S0 was given (the gradient with respect to the starting
    state)."""
    q, k, v, beta, dO = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(dO)
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if (q.shape != (B, H, L, d_k) or v.shape != (B, H, L, d_v) or dO.shape != (B, H, L, d_v)
            or beta.shape != (B, H, L)):
        raise ValueError("shape mismatch among q, k, v, beta, dO")
    S = np.zeros((B, H, d_k, d_v)) if S0 is None else _f64(S0).copy()
    if S.shape != (B, H, d_k, d_v):
        raise ValueError("S0 must be [B, H, d_k, d_v]")
    states = [S]
    for t in range(L):
        k_t = k[:, :, t, None, :]
        u_t = beta[:, :, t, None, None] * (v[:, :, t, None, :] - k_t @ S)
        S = S + np.swapaxes(k_t, -1, -2) @ u_t
        states.append(S)

    G = np.zeros((B, H, d_k, d_v)) if dS_final is None else _f64(dS_final).copy()
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dbeta = np.empty_like(beta)
    for t in range(L - 1, -1, -1):
        S_prev, S_t = states[t], states[t + 1]
        q_t, k_t = q[:, :, t, None, :], k[:, :, t, None, :]
        dO_t = dO[:, :, t, None, :]
        b = beta[:, :, t, None, None]
        G = G + np.swapaxes(q_t, -1, -2) @ dO_t
        dq[:, :, t] = (dO_t @ np.swapaxes(S_t, -1, -2))[:, :, 0]
        du = k_t @ G
        r_t = v[:, :, t, None, :] - k_t @ S_prev
        u_t = b * r_t
        dv[:, :, t] = (b * du)[:, :, 0]
        dbeta[:, :, t] = np.sum(du * r_t, axis=(-2, -1))
        dk[:, :, t] = (u_t @ np.swapaxes(G, -1, -2) - b * (du @ np.swapaxes(S_prev, -1, -2)))[:, :, 0]
        G = G - np.swapaxes(k_t, -1, -2) @ (b * du)
    return dq, dk, dv, dbeta, G
