"""Pins for the gated (Gated DeltaNet) oracle: facts fixed by the article and
by mathematics, each computed by a route that does not go through the token
loop.

Every ``gpin_*`` takes a gated forward callable
``fwd(q, k, v, alpha, beta, S0) -> (o, S_final)`` (fp64 numpy) and returns the
largest absolute deviation from the pinned values.  The article is "How a
Baseten Engineer Traced 7 Years of Attention Mechanism Evolution" (wpnews.pro,
canonical dev.to), section on Gated DeltaNet: the state is decayed by a scalar
alpha in [0, 1] first and then written with the precise delta; alpha = 1 is
the plain delta rule, alpha = 0 wipes the memory, and a value written at step
x and read at step x + t has been multiplied by the decays of the steps in
between.
"""

from __future__ import annotations

import functools

import numpy as np

from oracle import delta_rule_forward
from pins import _haar_orthogonal, _unit


def _inputs(rng, B, H, L, dk, dv, unit=True):
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    if unit:
        k = _unit(k)
    v = rng.standard_normal((B, H, L, dv))
    return q, k, v


def gpin_alpha_one_is_delta_rule(fwd, rng, B=2, H=2, L=13, dk=6, dv=5):
    """alpha = 1 is the plain delta rule (article), itself pinned separately."""
    q, k, v = _inputs(rng, B, H, L, dk, dv)
    beta = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, np.ones((B, H, L)), beta, S0)
    o2, S2 = delta_rule_forward(q, k, v, beta, S0)
    return max(np.abs(o - o2).max(), np.abs(S - S2).max())


def gpin_alpha_zero_wipes(fwd, rng, B=2, H=2, L=9, dk=5, dv=4):
    """alpha = 0 wipes the memory before each write, so only the current
    token's write survives: S_t = beta_t k_t^T v_t and o_t = beta_t (q_t . k_t) v_t.
    Keys are not orthogonal and S0 is random, so a delta that read the
    undecayed state would not pass."""
    q, k, v = _inputs(rng, B, H, L, dk, dv, unit=False)
    beta = rng.uniform(0.1, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, np.zeros((B, H, L)), beta, S0)
    want_o = (beta * np.einsum("bhld,bhld->bhl", q, k))[..., None] * v
    want_S = beta[:, :, -1, None, None] * k[:, :, -1, :, None] * v[:, :, -1, None, :]
    return max(np.abs(o - want_o).max(), np.abs(S - want_S).max())


def gpin_decay_only(fwd, rng, B=2, H=3, L=11, dk=4, dv=6):
    """beta = 0 turns the writes off, leaving the cumulative decay of the
    article: S_t = (alpha_1 ... alpha_t) S0 and o_t = (alpha_1 ... alpha_t) q_t S0."""
    q, k, v = _inputs(rng, B, H, L, dk, dv)
    alpha = rng.uniform(0.2, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, alpha, np.zeros((B, H, L)), S0)
    g = np.cumprod(alpha, axis=-1)
    want_o = g[..., None] * (q @ S0)
    want_S = g[:, :, -1, None, None] * S0
    return max(np.abs(o - want_o).max(), np.abs(S - want_S).max())


def gpin_gated_linear_attention(fwd, rng, B=2, H=2, dk=16, dv=7, L=12):
    """Orthonormal keys and S0 = 0: no read sees another key's write, so every
    delta is beta_r v_r and each write reaches a later read through the decays
    of the steps after it:
        o_r = sum_{i <= r} (alpha_{i+1} ... alpha_r) (q_r . k_i) beta_i v_i,
    i.e. masked linear attention with the decay mask (diagonal included)."""
    err = 0.0
    for b in range(B):
        for h in range(H):
            K = _haar_orthogonal(rng, dk)[:L]
            Q = rng.standard_normal((L, dk))
            V = rng.standard_normal((L, dv))
            beta = rng.uniform(0.0, 1.0, L)
            alpha = rng.uniform(0.3, 1.0, L)
            D = np.zeros((L, L))
            for r in range(L):
                for i in range(r + 1):
                    D[r, i] = np.prod(alpha[i + 1:r + 1])
            want = ((Q @ K.T) * D) @ (beta[:, None] * V)
            want_S = K.T @ ((D[L - 1][:, None] * beta[:, None]) * V)
            o, S = fwd(Q[None, None], K[None, None], V[None, None], alpha[None, None],
                       beta[None, None], None)
            err = max(err, np.abs(o[0, 0] - want).max(), np.abs(S[0, 0] - want_S).max())
    return err


def gpin_transition_product(fwd, rng, B=2, H=2, L=7, dk=5, dv=3):
    """Unrolled with explicit d_k x d_k matrices: decaying then writing makes
    the transition alpha_r P_r with P_r = I - beta_r k_r^T k_r, so
        S_t = (a_t P_t ... a_1 P_1) S0 + sum_{r<=t} (a_t P_t ... a_{r+1} P_{r+1}) beta_r k_r^T v_r.
    Keys are not normalised and d_k != d_v."""
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk)) * 0.6
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0.0, 1.0, (B, H, L))
    alpha = rng.uniform(0.0, 1.0, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, alpha, beta, S0)
    I = np.eye(dk)
    err = 0.0
    for b in range(B):
        for h in range(H):
            M = [alpha[b, h, r] * (I - beta[b, h, r] * np.outer(k[b, h, r], k[b, h, r]))
                 for r in range(L)]

            def chain(lo, hi):  # M_hi ... M_lo (1-based inclusive); identity if empty
                mats = [M[r - 1] for r in range(hi, lo - 1, -1)]
                return functools.reduce(np.matmul, mats, I)

            for t in range(1, L + 1):
                St = chain(1, t) @ S0[b, h]
                for r in range(1, t + 1):
                    St = St + chain(r + 1, t) @ (beta[b, h, r - 1] * np.outer(k[b, h, r - 1], v[b, h, r - 1]))
                err = max(err, np.abs(q[b, h, t - 1] @ St - o[b, h, t - 1]).max())
            err = max(err, np.abs(St - S[b, h]).max())
    return err


def gpin_scalar(fwd, rng, L=40):
    """d_k = d_v = 1 with k_t = +-1: s_t = alpha_t (1 - beta_t) s_{t-1} + beta_t k_t v_t."""
    k = rng.choice([-1.0, 1.0], L)
    v, q = rng.standard_normal(L), rng.standard_normal(L)
    beta, alpha = rng.uniform(0.0, 1.0, L), rng.uniform(0.0, 1.0, L)
    s = s0 = -0.4
    want = []
    for t in range(L):
        s = alpha[t] * (1.0 - beta[t]) * s + beta[t] * k[t] * v[t]
        want.append(q[t] * s)
    r = lambda x: x.reshape(1, 1, L)
    o, S = fwd(q.reshape(1, 1, L, 1), k.reshape(1, 1, L, 1), v.reshape(1, 1, L, 1), r(alpha),
               r(beta), np.full((1, 1, 1, 1), s0))
    return max(np.abs(o[0, 0, :, 0] - np.array(want)).max(), abs(S[0, 0, 0, 0] - s))


ALL_GATED_PINS = [
    gpin_alpha_one_is_delta_rule,
    gpin_alpha_zero_wipes,
    gpin_decay_only,
    gpin_gated_linear_attention,
    gpin_transition_product,
    gpin_scalar,
]
