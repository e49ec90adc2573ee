"""fp64 CPU oracle for the DeltaNet delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path: no kernels, headers, helpers or tables.  It is deliberately
plain and slow: one Python loop over tokens, vectorised over (batch, head)
only, no chunking, no reordering.

What it computes, and where the pages define it (all citations are to the
page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説", news.ainew.jp, unless
noted):

* ``delta_rule_forward`` follows the sequential delta-rule prefill loop in the
  section "DeltaNet (Parallelizing linear transformers with delta rule)": the
  state starts at zero (or at a given cache), and for each token i in order it
  reads the value the state holds at key k_i (v_old = k_i S), forms the gated
  delta u_i = beta_i (v_i - v_old), writes S <- S + k_i^T u_i, and then reads
  the output o_i = q_i S from the state *after* that write.
* ``delta_rule_decode_step`` is the layer forward of the section "DeltaNet
  (Fast weight programmers)" taken at one token (t = 1): read v_old = k S,
  u = beta (v - v_old), S <- S + k^T u, o = q S with no denominator.  The
  article "How a Baseten Engineer Traced 7 Years of Attention Mechanism
  Evolution" (wpnews.pro / dev.to), section on DeltaNet, states the same
  three-line update without beta (beta = 1).

Readings taken where the pages are silent (each listed in the design notes):
no 1/sqrt(d) scale on q; q and k are used as given (the feature map and the
normalisation sit before this core); beta is per (batch, head, token); the
state is d_k x d_v with the row-vector convention (v_old = k S); the output
is read after the write; a length that is not a multiple of any chunk size is
simply run token by token.

* ``gated_delta_rule_forward`` / ``gated_delta_rule_decode_step`` add the
  scalar gate of Gated DeltaNet from the article "How a Baseten Engineer
  Traced 7 Years of Attention Mechanism Evolution", section on Gated DeltaNet:
  the old state is first decayed by alpha_t in [0, 1] and the precise delta
  write then acts on the decayed state:
      S <- alpha_t S;  v_old = k_t S;  u_t = beta_t (v_t - v_old);
      S <- S + k_t^T u_t;  o_t = q_t S.
  alpha = 1 is the plain delta rule and alpha = 0 wipes the memory before the
  write (both as the article states).  Reading taken: the delta reads the
  decayed state ("decay first, then precise write").

Pins (tests/test_oracle_pins.py) tie this oracle to facts other than
itself: beta = 0 leaves the state alone; v_t = k_t S leaves it alone; with
beta = 1 and orthonormal keys the state returns the latest value written at a
key; with orthonormal keys the result collapses to masked linear attention
with V scaled by beta; an explicitly multiplied product of generalised
Householder transition matrices on tiny inputs; the scalar (d = 1) case as an
exponential moving average; and a hand-derived worked example under
tests/golden/.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def delta_rule_forward(q, k, v, beta, S0: Optional[np.ndarray] = None
                       ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token delta-rule forward in fp64.

    q, k: ``[B, H, L, d_k]``; v: ``[B, H, L, d_v]``; beta: ``[B, H, L]``;
    S0: ``[B, H, d_k, d_v]`` or None (zero state).

    Returns ``(o, S_final)`` with o ``[B, H, L, d_v]`` and S_final
    ``[B, H, d_k, d_v]``, both float64.
    """
    q, k, v, beta = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(beta)
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if q.shape != (B, H, L, d_k) or v.shape[:3] != (B, H, L) or beta.shape != (B, H, L):
        raise ValueError("shape mismatch among q, k, v, beta")
    if S0 is None:
        S = np.zeros((B, H, d_k, d_v))
    else:
        S = _as_f64(S0).copy()
        if S.shape != (B, H, d_k, d_v):
            raise ValueError("S0 must be [B, H, d_k, d_v]")
    o = np.empty((B, H, L, d_v))
    for t in range(L):
        k_t = k[:, :, t, None, :]                     # [B,H,1,d_k] row vector
        v_old = k_t @ S                               # read the state at key k_t
        u_t = beta[:, :, t, None, None] * (v[:, :, t, None, :] - v_old)
        S = S + np.swapaxes(k_t, -1, -2) @ u_t         # outer-product write k_t^T u_t
        o[:, :, t, :] = (q[:, :, t, None, :] @ S)[:, :, 0, :]  # read after the write
    return o, S


def delta_rule_decode_step(q, k, v, beta, S) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step in fp64 (the layer forward at a single token).

    q, k: ``[B, H, d_k]``; v: ``[B, H, d_v]``; beta: ``[B, H]``;
    S: ``[B, H, d_k, d_v]``.  Returns ``(o, S_new)``; S is not modified.
    """
    q, k, v, beta, S = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(beta), _as_f64(S)
    k_row = k[:, :, None, :]
    v_old = k_row @ S
    u = beta[:, :, None, None] * (v[:, :, None, :] - v_old)
    S_new = S + np.swapaxes(k_row, -1, -2) @ u
    o = (q[:, :, None, :] @ S_new)[:, :, 0, :]
    return o, S_new


def gated_delta_rule_forward(q, k, v, alpha, beta, S0: Optional[np.ndarray] = None
                             ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token gated delta-rule forward in fp64 (decay, then the delta
    write on the decayed state, then the read).

    alpha: ``[B, H, L]`` per-token decay in [0, 1]; the other arguments and
    the result are as in ``delta_rule_forward``.
    """
    q, k, v, beta, alpha = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(beta), _as_f64(alpha)
    B, H, L, d_k = k.shape
    d_v = v.shape[-1]
    if (q.shape != (B, H, L, d_k) or v.shape[:3] != (B, H, L) or beta.shape != (B, H, L)
            or alpha.shape != (B, H, L)):
        raise ValueError("shape mismatch among q, k, v, alpha, beta")
    if S0 is None:
        S = np.zeros((B, H, d_k, d_v))
    else:
        S = _as_f64(S0).copy()
        if S.shape != (B, H, d_k, d_v):
            raise ValueError("S0 must be [B, H, d_k, d_v]")
    o = np.empty((B, H, L, d_v))
    for t in range(L):
        S = alpha[:, :, t, None, None] * S                # decay first
        k_t = k[:, :, t, None, :]
        v_old = k_t @ S                                   # read the decayed state
        u_t = beta[:, :, t, None, None] * (v[:, :, t, None, :] - v_old)
        S = S + np.swapaxes(k_t, -1, -2) @ u_t            # precise write
        o[:, :, t, :] = (q[:, :, t, None, :] @ S)[:, :, 0, :]
    return o, S


def gated_delta_rule_decode_step(q, k, v, alpha, beta, S) -> Tuple[np.ndarray, np.ndarray]:
    """One gated decode step in fp64: the gated forward at a single token.

    alpha, beta: ``[B, H]``; the rest as in ``delta_rule_decode_step``.
    """
    q, k, v, beta, alpha, S = (_as_f64(q), _as_f64(k), _as_f64(v), _as_f64(beta),
                               _as_f64(alpha), _as_f64(S))
    S = alpha[:, :, None, None] * S
    k_row = k[:, :, None, :]
    u = beta[:, :, None, None] * (v[:, :, None, :] - k_row @ S)
    S_new = S + np.swapaxes(k_row, -1, -2) @ u
    o = (q[:, :, None, :] @ S_new)[:, :, 0, :]
    return o, S_new
