"""Pins for the backward oracle (oracle/backward.py) and planted mistakes.

The gradient of the delta-rule loop is fixed by calculus: the pins compare
the oracle's reverse pass with central finite differences of the forward
oracle (itself pinned in test_oracle_pins.py), with a closed form at
beta = 0, and with a hand-derived single token.  A loss L = sum(W_o * o) +
sum(W_S * S_final) has dO = W_o and dS_final = W_S.
"""

import numpy as np
import pytest

from oracle import delta_rule_backward, delta_rule_forward

TOL_FD = 1e-7    # central differences at h = 1e-5 in fp64: error O(h^2) + rounding
TOL = 1e-12


def _case(rng, B=1, H=2, L=7, dk=4, dv=3, s0=True):
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk)) * 0.5
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0.1, 0.9, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    Wo = rng.standard_normal((B, H, L, dv))
    WS = rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, S0, Wo, WS


def _loss(q, k, v, beta, S0, Wo, WS):
    o, S = delta_rule_forward(q, k, v, beta, S0)
    return float(np.sum(Wo * o) + np.sum(WS * S))


def pin_finite_differences(bwd, rng):
    """Every gradient against central differences of the forward oracle."""
    q, k, v, beta, S0, Wo, WS = _case(rng)
    grads = bwd(q, k, v, beta, S0, Wo, WS)
    args = [q, k, v, beta, S0]
    h = 1e-5
    err = 0.0
    for idx, (x, g) in enumerate(zip(args, grads)):
        flat = x.reshape(-1)
        for n in range(flat.size):
            keep = flat[n]
            flat[n] = keep + h
            lp = _loss(*args, Wo, WS)
            flat[n] = keep - h
            lm = _loss(*args, Wo, WS)
            flat[n] = keep
            fd = (lp - lm) / (2 * h)
            err = max(err, abs(fd - g.reshape(-1)[n]) / max(1.0, abs(fd)))
    return err / TOL_FD * TOL  # scaled so that the common bar TOL applies


def pin_beta_zero_closed_form(bwd, rng):
    """beta = 0: o_t = q_t S0 for every t and S_final = S0, so
    dq_t = dO_t S0^T, dS0 = dS_final + sum_t q_t^T dO_t, dv = dk = 0, and
    dbeta_t = (k_t G_t) . (v_t - k_t S0) with G_t = dS_final + sum_{s >= t} q_s^T dO_s."""
    q, k, v, _, S0, Wo, WS = _case(rng, L=6)
    beta = np.zeros(q.shape[:3])
    dq, dk, dv, db, dS0 = bwd(q, k, v, beta, S0, Wo, WS)
    want_dq = np.einsum("bhle,bhde->bhld", Wo, S0)
    QtdO = np.einsum("bhld,bhle->bhlde", q, Wo)
    G = WS[:, :, None] + np.flip(np.cumsum(np.flip(QtdO, 2), axis=2), 2)   # [B,H,L,dk,dv]
    r = v - np.einsum("bhld,bhde->bhle", k, S0)
    want_db = np.einsum("bhld,bhlde,bhle->bhl", k, G, r)
    return max(np.abs(dq - want_dq).max(), np.abs(dk).max(), np.abs(dv).max(),
               np.abs(db - want_db).max(), np.abs(dS0 - (WS + QtdO.sum(axis=2))).max())


def pin_single_token(bwd, rng):
    """L = 1 by hand: S1 = S0 + b k^T (v - k S0), o = q S1.  With G = dS_final
    + q^T dO and du = k G: dq = dO S1^T, dv = b du, dbeta = du . (v - k S0),
    dk = b (v - k S0) G^T - b du S0^T, dS0 = G - b k^T du."""
    q, k, v, beta, S0, Wo, WS = _case(rng, L=1)
    dq, dk, dv, db, dS0 = bwd(q, k, v, beta, S0, Wo, WS)
    err = 0.0
    for b_ in range(q.shape[0]):
        for h in range(q.shape[1]):
            qq, kk, vv, bb = q[b_, h, 0], k[b_, h, 0], v[b_, h, 0], beta[b_, h, 0]
            s0, dO, dSf = S0[b_, h], Wo[b_, h, 0], WS[b_, h]
            r = vv - kk @ s0
            S1 = s0 + bb * np.outer(kk, r)
            G = dSf + np.outer(qq, dO)
            du = kk @ G
            err = max(err, np.abs(dq[b_, h, 0] - S1 @ dO).max(),
                      np.abs(dv[b_, h, 0] - bb * du).max(),
                      abs(db[b_, h, 0] - du @ r),
                      np.abs(dk[b_, h, 0] - (bb * G @ r - bb * s0 @ du)).max(),
                      np.abs(dS0[b_, h] - (G - bb * np.outer(kk, du))).max())
    return err


BWD_PINS = [pin_finite_differences, pin_beta_zero_closed_form, pin_single_token]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    assert pin(delta_rule_backward, np.random.default_rng(21)) < TOL


def test_backward_without_S0_and_dS_final():
    """None means zero for both; the result equals passing zeros."""
    rng = np.random.default_rng(22)
    q, k, v, beta, _, Wo, _ = _case(rng, s0=False)
    a = delta_rule_backward(q, k, v, beta, None, Wo, None)
    z = np.zeros((1, 2, 4, 3))
    b = delta_rule_backward(q, k, v, beta, z, Wo, z)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# --- planted mistakes -----------------------------------------------------

def _mutant(mutant):
    def bwd(q, k, v, beta, S0, dO, dSf):
        q, k, v, beta, dO = (np.asarray(x, float) for x in (q, k, v, beta, dO))
        B, H, L, dk_ = k.shape
        dv_ = v.shape[-1]
        S = np.zeros((B, H, dk_, dv_)) if S0 is None else np.asarray(S0, float).copy()
        states = [S]
        for t in range(L):
            kt = k[:, :, t, None, :]
            u = beta[:, :, t, None, None] * (v[:, :, t, None, :] - kt @ S)
            S = S + np.swapaxes(kt, -1, -2) @ u
            states.append(S)
        G = np.zeros((B, H, dk_, dv_)) if dSf is None else np.asarray(dSf, float).copy()
        dq, dk, dv, db = (np.empty_like(x) for x in (q, k, v, beta))
        for t in range(L - 1, -1, -1):
            Sp, St = states[t], states[t + 1]
            qt, kt, dOt = q[:, :, t, None, :], k[:, :, t, None, :], dO[:, :, t, None, :]
            b = beta[:, :, t, None, None]
            if mutant != "read_grad_after_du":
                G = G + np.swapaxes(qt, -1, -2) @ dOt
            dq[:, :, t] = (dOt @ np.swapaxes(Sp if mutant == "dq_uses_old_state" else St, -1, -2))[:, :, 0]
            du = kt @ G
            if mutant == "read_grad_after_du":
                G = G + np.swapaxes(qt, -1, -2) @ dOt
            r = v[:, :, t, None, :] - kt @ Sp
            dv[:, :, t] = (du if mutant == "dv_without_beta" else b * du)[:, :, 0]
            db[:, :, t] = np.sum(du * (v[:, :, t, None, :] if mutant == "dbeta_uses_v" else r), axis=(-2, -1))
            dk_t = b * r @ np.swapaxes(G, -1, -2)
            if mutant != "dk_missing_read_term":
                dk_t = dk_t - b * (du @ np.swapaxes(Sp, -1, -2))
            dk[:, :, t] = dk_t[:, :, 0]
            if mutant == "no_state_grad_through_delta":
                continue
            G = G - np.swapaxes(kt, -1, -2) @ ((b if mutant != "transition_sign" else -b) * du)
        return dq, dk, dv, db, G
    return bwd


BWD_MUTANTS = ["read_grad_after_du", "dq_uses_old_state", "dv_without_beta", "dbeta_uses_v",
               "dk_missing_read_term", "no_state_grad_through_delta", "transition_sign"]


def test_unmutated_backward_copy_passes_every_pin():
    for pin in BWD_PINS:
        assert pin(_mutant(None), np.random.default_rng(21)) < TOL, pin.__name__


@pytest.mark.parametrize("mutant", BWD_MUTANTS)
def test_backward_mutant_is_caught(mutant):
    caught = [p.__name__ for p in BWD_PINS if not p(_mutant(mutant), np.random.default_rng(21)) < TOL]
    assert caught, f"mutant {mutant!r} passed every pin"
