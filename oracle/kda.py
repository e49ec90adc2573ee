"""fp64 CPU oracle for the delta rule with per-dimension decay (KDA).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path: a plain Python loop over tokens, vectorised over (batch, head).

What it computes.  The article "How a Baseten Engineer Traced 7 Years of
Attention Mechanism Evolution" (wpnews.pro / dev.to) describes Kimi Linear's
KDA as the step from Gated DeltaNet's single scalar gate to a gate per
dimension: alpha becomes a vector, and each dimension of the memory forgets
at its own rate.  Gated DeltaNet, in the same article, decays the old state
first and then applies the precise delta write.  With the state S a
d_k x d_v matrix read as v_old = k S, the dimensions a key addresses are the
rows of S, so per token t, in order:
    S     <- diag(alpha_t) S          alpha_t in [0, 1]^{d_k}
    v_old  = k_t S                    (the decayed state)
    u_t    = beta_t (v_t - v_old)
    S     <- S + k_t^T u_t
    o_t    = q_t S

Readings taken (listed in the design notes): alpha_t is a d_k-vector acting
on the key dimension (the rows of S); a gate that is a full matrix, which the
article also allows, is not taken; the decay comes before the write, and the
delta reads the decayed state, as for the scalar gate.

Pins (tests/test_oracle_kda.py): a constant vector reduces to the scalar gated
oracle (itself pinned) and all-ones to the plain delta rule; beta = 0 leaves
only the per-row decay products; coordinate keys give a closed-form masked
linear attention with per-dimension decay; an explicit product of
transition matrices diag(alpha) - beta k^T (k diag(alpha)) at tiny sizes; keys
confined to a block of coordinates leave the other rows to decay alone; and
planted mistakes (decay on the value dimension, decay after the write, the
previous token's gate, the mean gate, a delta that reads the undecayed state)
that each fail one of them.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def kda_delta_rule_forward(q, k, v, alpha, beta, S0: Optional[np.ndarray] = None
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token forward with per-dimension decay, fp64.

    q, k: ``[B, H, L, d_k]``; v: ``[B, H, L, d_v]``; alpha: ``[B, H, L, d_k]``
    in [0, 1]; beta: ``[B, H, L]``; S0: ``[B, H, d_k, d_v]`` or None (zero).
    Returns (o ``[B, H, L, d_v]``, S_final ``[B, H, d_k, d_v]``).
    """
    q, k, v, alpha, beta = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta)
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if (q.shape != (B, H, L, d_k) or v.shape[:3] != (B, H, L) or beta.shape != (B, H, L)
            or alpha.shape != (B, H, L, d_k)):
        raise ValueError("shape mismatch among q, k, v, alpha, beta")
    S = np.zeros((B, H, d_k, d_v)) if S0 is None else _f64(S0).copy()
    if S.shape != (B, H, d_k, d_v):
        raise ValueError("S0 must be [B, H, d_k, d_v]")
    o = np.empty((B, H, L, d_v))
    for t in range(L):
        S = alpha[:, :, t, :, None] * S                   # row j of S decays by alpha_t[j]
        k_t = k[:, :, t, None, :]
        u_t = beta[:, :, t, None, None] * (v[:, :, t, None, :] - k_t @ S)
        S = S + np.swapaxes(k_t, -1, -2) @ u_t
        o[:, :, t, :] = (q[:, :, t, None, :] @ S)[:, :, 0, :]
    return o, S


def kda_delta_rule_decode_step(q, k, v, alpha, beta, S) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step with per-dimension decay: the forward at one token.

    q, k, alpha: ``[B, H, d_k]``; v: ``[B, H, d_v]``; beta: ``[B, H]``;
    S: ``[B, H, d_k, d_v]``.  Returns (o ``[B, H, d_v]``, S_new).
    """
    q, k, v, alpha, beta, S = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(beta), _f64(S)
    S = alpha[:, :, :, None] * S
    k_row = k[:, :, None, :]
    u = beta[:, :, None, None] * (v[:, :, None, :] - k_row @ S)
    S_new = S + np.swapaxes(k_row, -1, -2) @ u
    o = (q[:, :, None, :] @ S_new)[:, :, 0, :]
    return o, S_new
