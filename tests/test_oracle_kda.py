"""Pins for the per-dimension-decay (KDA) oracle, oracle/kda.py, and planted
mistakes that each of them must catch.

The article "How a Baseten Engineer Traced 7 Years of Attention Mechanism
Evolution" (wpnews.pro / dev.to) describes KDA as Gated DeltaNet with the
scalar gate alpha turned into a vector, one forgetting rate per memory
dimension; the gated step decays first and then writes the precise delta.
Every ``kpin_*`` takes a forward ``fwd(q, k, v, alpha, beta, S0) -> (o, S)``
(alpha ``[B, H, L, d_k]``) and returns the largest deviation from values
computed by another route.
"""

import numpy as np
import pytest

from oracle import (delta_rule_forward, gated_delta_rule_forward, kda_delta_rule_decode_step,
                    kda_delta_rule_forward)
from pins import _unit

TOL = 1e-12


def _qkv(rng, B, H, L, dk, dv, unit=True):
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    return q, (_unit(k) if unit else k), v


def kpin_ones_is_delta_rule(fwd, rng, B=2, H=2, L=11, dk=6, dv=5):
    """All-ones gates are the plain delta rule (pinned on its own)."""
    q, k, v = _qkv(rng, B, H, L, dk, dv)
    beta = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, np.ones((B, H, L, dk)), beta, S0)
    o2, S2 = delta_rule_forward(q, k, v, beta, S0)
    return max(np.abs(o - o2).max(), np.abs(S - S2).max())


def kpin_constant_vector_is_scalar_gate(fwd, rng, B=2, H=2, L=12, dk=5, dv=7):
    """A gate equal in every dimension is Gated DeltaNet's scalar gate (its
    oracle is pinned on its own)."""
    q, k, v = _qkv(rng, B, H, L, dk, dv)
    beta = rng.uniform(0, 1, (B, H, L))
    a = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, np.repeat(a[..., None], dk, axis=-1), beta, S0)
    o2, S2 = gated_delta_rule_forward(q, k, v, a, beta, S0)
    return max(np.abs(o - o2).max(), np.abs(S - S2).max())


def kpin_decay_only(fwd, rng, B=2, H=2, L=10, dk=4, dv=6):
    """beta = 0: no writes, so S_t = diag(alpha_1 ... alpha_t) S0 row by row
    and o_t = q_t S_t."""
    q, k, v = _qkv(rng, B, H, L, dk, dv)
    a = rng.uniform(0.3, 1, (B, H, L, dk))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, a, np.zeros((B, H, L)), S0)
    prod = np.cumprod(a, axis=2)                                   # [B,H,L,dk]
    want_o = np.einsum("bhld,bhde->bhle", q * prod, S0)
    want_S = prod[:, :, -1, :, None] * S0
    return max(np.abs(o - want_o).max(), np.abs(S - want_S).max())


def kpin_coordinate_keys(fwd, rng, B=1, H=2, dk=6, dv=6):
    """Keys that are distinct coordinate vectors e_{a_t}, from the zero state:
    every read of a fresh key finds zero, so u_t = beta_t v_t, and
        o_t = sum_{i <= t} q_t[a_i] (prod_{i < m <= t} alpha_m[a_i]) beta_i v_i,
    masked linear attention with each write decaying in its own dimension.
    Then, with beta = 1, writing a used coordinate again overwrites it: the
    state's row for it equals the latest value whatever decayed before."""
    L = dk
    perm = rng.permutation(dk)
    k = np.zeros((B, H, L, dk))
    k[:, :, np.arange(L), perm] = 1.0
    q = rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    a = rng.uniform(0.2, 1, (B, H, L, dk))
    beta = rng.uniform(0.1, 1, (B, H, L))
    o, _ = fwd(q, k, v, a, beta, None)
    want = np.zeros((B, H, L, dv))
    for t in range(L):
        for i in range(t + 1):
            dec = np.prod(a[:, :, i + 1:t + 1, perm[i]], axis=2)     # [B,H]
            want[:, :, t] += (q[:, :, t, perm[i]] * dec * beta[:, :, i])[..., None] * v[:, :, i]
    err = np.abs(o - want).max()
    # overwrite: keys e_0, e_1, e_0 with beta = 1
    k2 = np.zeros((B, H, 3, dk))
    k2[:, :, [0, 2], 0] = 1.0
    k2[:, :, 1, 1] = 1.0
    v2 = rng.standard_normal((B, H, 3, dv))
    a2 = rng.uniform(0.2, 1, (B, H, 3, dk))
    _, S2 = fwd(rng.standard_normal((B, H, 3, dk)), k2, v2, a2, np.ones((B, H, 3)), None)
    return max(err, np.abs(S2[:, :, 0] - v2[:, :, 2]).max(),
               np.abs(S2[:, :, 1] - a2[:, :, 2, 1, None] * v2[:, :, 1]).max())


def kpin_transition_product(fwd, rng, B=1, H=2, L=6, dk=4, dv=3):
    """Unrolled: S_t = M_t S_{t-1} + beta_t k_t^T v_t with the transition
    M_t = (I - beta_t k_t^T k_t) diag(alpha_t), multiplied out explicitly."""
    q, k, v = _qkv(rng, B, H, L, dk, dv, unit=False)
    beta = rng.uniform(0, 1, (B, H, L))
    a = rng.uniform(0, 1, (B, H, L, dk))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = fwd(q, k, v, a, beta, S0)
    err = 0.0
    for b in range(B):
        for h in range(H):
            M = [(np.eye(dk) - beta[b, h, t] * np.outer(k[b, h, t], k[b, h, t])) @ np.diag(a[b, h, t])
                 for t in range(L)]
            W = [beta[b, h, t] * np.outer(k[b, h, t], v[b, h, t]) for t in range(L)]
            for t in range(L):
                Phi = np.eye(dk)
                for m in range(t, -1, -1):
                    Phi = Phi @ M[m]
                St = Phi @ S0[b, h]
                for i in range(t + 1):
                    P = np.eye(dk)
                    for m in range(t, i, -1):
                        P = P @ M[m]
                    St = St + P @ W[i]
                err = max(err, np.abs(q[b, h, t] @ St - o[b, h, t]).max())
            err = max(err, np.abs(St - S[b, h]).max())
    return err


def kpin_untouched_rows_only_decay(fwd, rng, B=2, H=2, L=9, dk=6, dv=4):
    """Keys confined to the first half of the coordinates never read or write
    the other rows of the state: those rows only decay, row j by the product
    of alpha_t[j]."""
    q, k, v = _qkv(rng, B, H, L, dk, dv, unit=False)
    k[..., dk // 2:] = 0.0
    a = rng.uniform(0.3, 1, (B, H, L, dk))
    beta = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv))
    _, S = fwd(q, k, v, a, beta, S0)
    prod = np.prod(a[..., dk // 2:], axis=2)
    return np.abs(S[:, :, dk // 2:] - prod[..., None] * S0[:, :, dk // 2:]).max()


def kpin_scalar(fwd, rng, B=2, H=2, L=15):
    """d_k = d_v = 1: s_t = alpha_t (1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t."""
    q, k, v = (rng.standard_normal((B, H, L, 1)) for _ in range(3))
    a = rng.uniform(0, 1, (B, H, L, 1))
    beta = rng.uniform(0, 1, (B, H, L))
    s = rng.standard_normal((B, H))
    o, S = fwd(q, k, v, a, beta, s[..., None, None])
    err = 0.0
    for t in range(L):
        kt, vt = k[:, :, t, 0], v[:, :, t, 0]
        s = a[:, :, t, 0] * (1 - beta[:, :, t] * kt * kt) * s + beta[:, :, t] * kt * vt
        err = max(err, np.abs(o[:, :, t, 0] - q[:, :, t, 0] * s).max())
    return max(err, np.abs(S[..., 0, 0] - s).max())


KDA_PINS = [kpin_ones_is_delta_rule, kpin_constant_vector_is_scalar_gate, kpin_decay_only,
            kpin_coordinate_keys, kpin_transition_product, kpin_untouched_rows_only_decay,
            kpin_scalar]


@pytest.mark.parametrize("pin", KDA_PINS, ids=lambda p: p.__name__)
def test_kda_oracle_pin(pin):
    assert pin(kda_delta_rule_forward, np.random.default_rng(11)) < TOL


def test_kda_decode_step_is_forward_at_one_token():
    rng = np.random.default_rng(12)
    B, H, dk, dv, T = 2, 3, 5, 4, 6
    q, k, v = _qkv(rng, B, H, T, dk, dv)
    a = rng.uniform(0, 1, (B, H, T, dk))
    beta = rng.uniform(0, 1, (B, H, T))
    S = rng.standard_normal((B, H, dk, dv))
    o_f, S_f = kda_delta_rule_forward(q, k, v, a, beta, S)
    for t in range(T):
        o_t, S = kda_delta_rule_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t],
                                            beta[:, :, t], S)
        assert np.abs(o_t - o_f[:, :, t]).max() < 1e-13
    assert np.abs(S - S_f).max() < 1e-13


# --- planted mistakes (copies of the loop on the CPU) ---------------------

def _mutant(mutant):
    def fwd(q, k, v, a, beta, S0):
        q, k, v, a, beta = (np.asarray(x, float) for x in (q, k, v, a, beta))
        B, H, L, dk = k.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.asarray(S0, float).copy()
        o = np.empty((B, H, L, dv))
        for t in range(L):
            at = a[:, :, t]
            if mutant == "previous_gate":
                at = a[:, :, t - 1] if t > 0 else np.ones_like(at)
            if mutant == "mean_gate":
                at = np.repeat(at.mean(axis=-1, keepdims=True), dk, axis=-1)
            if mutant == "value_dim_decay":
                Sd = at[:, :, None, :] * S
            elif mutant == "no_decay_of_S0" and t == 0:
                Sd = S
            else:
                Sd = at[:, :, :, None] * S
            kt = k[:, :, t, None, :]
            read = kt @ (S if mutant == "delta_reads_undecayed" else Sd)
            u = beta[:, :, t, None, None] * (v[:, :, t, None, :] - read)
            if mutant == "decay_after_write":
                S = at[:, :, :, None] * (S + np.swapaxes(kt, -1, -2) @ (
                    beta[:, :, t, None, None] * (v[:, :, t, None, :] - kt @ S)))
            elif mutant == "decay_the_write_too":
                S = Sd + at[:, :, :, None] * (np.swapaxes(kt, -1, -2) @ u)
            else:
                S = Sd + np.swapaxes(kt, -1, -2) @ u
            o[:, :, t] = (q[:, :, t, None, :] @ S)[:, :, 0, :]
        return o, S

    return fwd


KDA_MUTANTS = ["previous_gate", "mean_gate", "value_dim_decay", "no_decay_of_S0",
               "delta_reads_undecayed", "decay_after_write", "decay_the_write_too"]


def test_unmutated_kda_copy_passes_every_pin():
    for pin in KDA_PINS:
        assert pin(_mutant(None), np.random.default_rng(11)) < TOL, pin.__name__


@pytest.mark.parametrize("mutant", KDA_MUTANTS)
def test_kda_mutant_is_caught(mutant):
    caught = []
    for pin in KDA_PINS:
        try:
            err = pin(_mutant(mutant), np.random.default_rng(11))
        except (ValueError, IndexError):
            err = np.inf
        if not err < TOL:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant!r} passed every pin"
