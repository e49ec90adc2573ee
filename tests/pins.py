"""Pins for the delta-rule oracle: facts fixed by the pages and by mathematics,
each computed here by a route that does not go through the token loop.

Every ``pin_*`` function takes a forward callable
``fwd(q, k, v, beta, S0) -> (o, S_final)`` (fp64 numpy, shapes as in
``oracle.delta_rule_forward``) and returns the largest absolute deviation from
the pinned values.  The mutation tests feed deliberately broken copies of the
recurrence through the same functions to show each plausible mistake trips
at least one pin.

Citations: "ainew page" is "GPT-2 から Kimi K3 まで、AI モデルの進化を解説"
(news.ainew.jp); "wpnews article" is "How a Baseten Engineer Traced 7 Years of
Attention Mechanism Evolution" (wpnews.pro, canonical dev.to).
"""

from __future__ import annotations

import functools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_examples.json")


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _haar_orthogonal(rng, n):
    """Haar-random orthogonal n x n matrix (QR of a Gaussian, sign-fixed)."""
    a = rng.standard_normal((n, n))
    qm, r = np.linalg.qr(a)
    return qm * np.sign(np.diag(r))[None, :]


def pin_beta_zero(fwd, rng, B=2, H=3, L=11, dk=5, dv=4):
    """beta = 0 turns every write off: S stays S0 and o_t = q_t S0.
    (ainew page, "DeltaNet (Fast weight programmers)": beta is the per-token
    write strength.)"""
    q = rng.standard_normal((B, H, L, dk))
    k = _unit(rng.standard_normal((B, H, L, dk)))
    v = rng.standard_normal((B, H, L, dv))
    S0 = rng.standard_normal((B, H, dk, dv))
    beta = np.zeros((B, H, L))
    o, S = fwd(q, k, v, beta, S0)
    want_o = q @ S0
    return max(np.abs(o - want_o).max(), np.abs(S - S0).max())


def pin_zero_delta(fwd, rng, B=2, H=2, L=9, dk=6, dv=3):
    """If the new value equals what the state already holds at the key, the
    delta is zero and nothing changes (wpnews article, DeltaNet section).
    With v_t = k_t S0 for every t the state never moves, so o_t = q_t S0."""
    q = rng.standard_normal((B, H, L, dk))
    k = _unit(rng.standard_normal((B, H, L, dk)))
    S0 = rng.standard_normal((B, H, dk, dv))
    v = k @ S0
    beta = rng.uniform(0.05, 1.0, (B, H, L))
    o, S = fwd(q, k, v, beta, S0)
    return max(np.abs(o - q @ S0).max(), np.abs(S - S0).max())


def pin_overwrite_retrieval(fwd, rng, B=2, H=2, dk=8, dv=5):
    """beta = 1 with orthonormal keys: reading back any key written so far
    returns its value exactly (ainew page: unit keys make the read exact; the
    erase term is a projection).  Queries equal to earlier keys retrieve those
    keys' values; the final state maps each key to its value."""
    L = dk
    err = 0.0
    for b in range(B):
        for h in range(H):
            K = _haar_orthogonal(rng, dk)          # rows orthonormal
            V = rng.standard_normal((L, dv))
            # query t asks for a key written at or before t
            pick = np.array([rng.integers(0, t + 1) for t in range(L)])
            Q = K[pick]
            o, S = fwd(Q[None, None], K[None, None], V[None, None],
                       np.ones((1, 1, L)), None)
            err = max(err, np.abs(o[0, 0] - V[pick]).max())
            err = max(err, np.abs(K @ S[0, 0] - V).max())
    return err


def pin_repeated_key_overwrite(fwd, rng, dk=6, dv=4, L=10):
    """beta = 1 and a unit key: after the write, reading that key returns the
    new value whatever the state held before (the delta equals the new value
    minus the old read, so the old association is replaced).  Keys repeat
    and the state starts random; each step's own key must read back v_t."""
    keys = _unit(rng.standard_normal((3, dk)))
    idx = rng.integers(0, 3, L)
    K = keys[idx]
    V = rng.standard_normal((L, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    Q = K.copy()  # read back the key just written
    o, _ = fwd(Q[None, None], K[None, None], V[None, None], np.ones((1, 1, L)), S0)
    return np.abs(o[0, 0] - V).max()


def pin_linear_attention_reduction(fwd, rng, B=2, H=2, dk=16, dv=7, L=12):
    """With orthonormal keys and S0 = 0 no read ever sees an earlier write, so
    the delta rule reduces to causal linear attention with V scaled by beta:
    o = tril(Q K^T) diag(beta) V, diagonal included (the chunked linear
    attention form of the ainew page, "DeltaNet (Parallelizing ...)", at one
    chunk, and its masked, score-first order inside a chunk)."""
    err = 0.0
    for b in range(B):
        for h in range(H):
            K = _haar_orthogonal(rng, dk)[:L]
            Q = rng.standard_normal((L, dk))
            V = rng.standard_normal((L, dv))
            beta = rng.uniform(0.0, 1.0, L)
            want = np.tril(Q @ K.T) @ (beta[:, None] * V)
            want_S = K.T @ (beta[:, None] * V)
            o, S = fwd(Q[None, None], K[None, None], V[None, None], beta[None, None], None)
            err = max(err, np.abs(o[0, 0] - want).max(), np.abs(S[0, 0] - want_S).max())
    return err


def pin_householder_product(fwd, rng, B=2, H=2, L=7, dk=5, dv=3):
    """The recurrence is a first-order linear recurrence whose transition
    matrices are generalised Householder matrices P_r = I - beta_r k_r^T k_r
    (ainew page, "DeltaNet (Parallelizing ...)").  Unrolled:
        S_t = (P_t ... P_1) S0 + sum_{r<=t} (P_t ... P_{r+1}) beta_r k_r^T v_r.
    Every product is formed explicitly as a d_k x d_k matrix; keys are not
    normalised and d_k != d_v so a transposed operand cannot pass."""
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk)) * 0.6
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0.0, 1.0, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, beta, S0)
    I = np.eye(dk)
    err = 0.0
    for b in range(B):
        for h in range(H):
            P = [I - beta[b, h, r] * np.outer(k[b, h, r], k[b, h, r]) for r in range(L)]

            def chain(lo, hi):  # P_hi ... P_lo (1-based inclusive); identity if empty
                mats = [P[r - 1] for r in range(hi, lo - 1, -1)]
                return functools.reduce(np.matmul, mats, I)

            for t in range(1, L + 1):
                St = chain(1, t) @ S0[b, h]
                for r in range(1, t + 1):
                    St = St + chain(r + 1, t) @ (beta[b, h, r - 1] * np.outer(k[b, h, r - 1], v[b, h, r - 1]))
                err = max(err, np.abs(q[b, h, t - 1] @ St - o[b, h, t - 1]).max())
            err = max(err, np.abs(St - S[b, h]).max())
    return err


def pin_scalar_ema(fwd, rng, L=40):
    """d_k = d_v = 1 with k_t = +-1: the update becomes an exponential moving
    average s_t = (1 - beta_t) s_{t-1} + beta_t k_t v_t, and o_t = q_t s_t."""
    k = rng.choice([-1.0, 1.0], L)
    v = rng.standard_normal(L)
    q = rng.standard_normal(L)
    beta = rng.uniform(0.0, 1.0, L)
    s0 = 0.7
    s = s0
    want = []
    for t in range(L):
        s = (1.0 - beta[t]) * s + beta[t] * k[t] * v[t]
        want.append(q[t] * s)
    o, S = fwd(q.reshape(1, 1, L, 1), k.reshape(1, 1, L, 1), v.reshape(1, 1, L, 1),
               beta.reshape(1, 1, L), np.full((1, 1, 1, 1), s0))
    return max(np.abs(o[0, 0, :, 0] - np.array(want)).max(), abs(S[0, 0, 0, 0] - s))


def pin_golden(fwd, rng=None):
    """Hand-derived worked examples stored under tests/golden/."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    err = 0.0
    for c in cases:
        q = np.array(c["q"], float)[None, None]
        k = np.array(c["k"], float)[None, None]
        v = np.array(c["v"], float)[None, None]
        beta = np.array(c["beta"], float)[None, None]
        S0 = None if c["S0"] is None else np.array(c["S0"], float)[None, None]
        o, S = fwd(q, k, v, beta, S0)
        err = max(err, np.abs(o[0, 0] - np.array(c["o"])).max(),
                  np.abs(S[0, 0] - np.array(c["S_final"])).max())
    return err


ALL_PINS = [
    pin_beta_zero,
    pin_zero_delta,
    pin_overwrite_retrieval,
    pin_repeated_key_overwrite,
    pin_linear_attention_reduction,
    pin_householder_product,
    pin_scalar_ema,
    pin_golden,
]

# fp64 arithmetic on O(1) values over short sequences: a correct
# implementation lands within a few ulps; 1e-10 leaves room for reordering.
PIN_TOL = 1e-10
