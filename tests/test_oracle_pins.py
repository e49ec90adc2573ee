"""The fp64 oracle against facts other than itself (CPU only)."""

import numpy as np
import pytest

from oracle import delta_rule_decode_step, delta_rule_forward
from pins import ALL_PINS, PIN_TOL
from wy_model import chunked_forward, chunked_forward_wu, wy_T


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    rng = np.random.default_rng(1234)
    err = pin(delta_rule_forward, rng)
    assert err < PIN_TOL, f"{pin.__name__}: max deviation {err:.3e}"


def test_decode_step_is_forward_at_one_token():
    """The decode step (layer forward at t = 1) equals one token of the loop,
    and chaining steps equals the loop over the same tokens."""
    rng = np.random.default_rng(7)
    B, H, L, dk, dv = 3, 2, 6, 8, 5
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.1
    o_ref, S_ref = delta_rule_forward(q, k, v, beta, S0)
    S = S0
    for t in range(L):
        o_t, S = delta_rule_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], beta[:, :, t], S)
        assert np.abs(o_t - o_ref[:, :, t]).max() < 1e-12
    assert np.abs(S - S_ref).max() < 1e-12


def test_decode_step_identity():
    """o = q S_new = q S_old + (q . k) u, the single-read form the decode
    kernel uses, written out from the definitions."""
    rng = np.random.default_rng(8)
    B, H, dk, dv = 2, 3, 7, 4
    q, k = rng.standard_normal((B, H, dk)), rng.standard_normal((B, H, dk))
    v, beta = rng.standard_normal((B, H, dv)), rng.uniform(0, 1, (B, H))
    S = rng.standard_normal((B, H, dk, dv))
    o, S_new = delta_rule_decode_step(q, k, v, beta, S)
    r = np.einsum("bhk,bhkv->bhv", k, S)
    u = beta[..., None] * (v - r)
    o2 = np.einsum("bhk,bhkv->bhv", q, S) + np.einsum("bhk,bhk->bh", q, k)[..., None] * u
    assert np.abs(o - o2).max() < 1e-12
    assert np.abs(S_new - (S + k[..., :, None] * u[..., None, :])).max() < 1e-12


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        delta_rule_forward(np.zeros((1, 1, 4, 3)), np.zeros((1, 1, 4, 2)),
                           np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4)))
    with pytest.raises(ValueError):
        delta_rule_forward(np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)),
                           np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4)), np.zeros((1, 1, 3, 2)))


def test_oracle_empty_sequence():
    """L = 0: no token, the state passes through unchanged."""
    S0 = np.arange(6.0).reshape(1, 1, 2, 3)
    o, S = delta_rule_forward(np.zeros((1, 1, 0, 2)), np.zeros((1, 1, 0, 2)),
                              np.zeros((1, 1, 0, 3)), np.zeros((1, 1, 0)), S0)
    assert o.shape == (1, 1, 0, 3)
    assert np.array_equal(S, S0)


# ---- the chunked algebra the kernels implement, against the oracle --------

def _rand_head(rng, L, dk, dv, s0=True):
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    S0 = rng.standard_normal((dk, dv)) * 0.1 if s0 else None
    return q, k, v, beta, S0


@pytest.mark.parametrize("C", [1, 7, 16, 64, 100])
@pytest.mark.parametrize("L", [100, 130])
def test_wy_chunked_form_equals_recurrence(C, L):
    rng = np.random.default_rng(C * 1000 + L)
    q, k, v, beta, S0 = _rand_head(rng, L, 16, 12)
    o_ref, S_ref = delta_rule_forward(q[None, None], k[None, None], v[None, None],
                                      beta[None, None], S0[None, None])
    o, S = chunked_forward(q, k, v, beta, S0, C)
    assert np.abs(o - o_ref[0, 0]).max() < 1e-12
    assert np.abs(S - S_ref[0, 0]).max() < 1e-12
    o2, S2 = chunked_forward_wu(q, k, v, beta, S0, C)
    assert np.abs(o2 - o_ref[0, 0]).max() < 1e-12
    assert np.abs(S2 - S_ref[0, 0]).max() < 1e-12


def test_wy_T_is_inverse_and_lower_triangular():
    rng = np.random.default_rng(3)
    C, dk = 64, 32
    k = rng.standard_normal((C, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = rng.uniform(0, 1, C)
    T = wy_T(k, beta)
    A = np.tril(beta[:, None] * (k @ k.T), -1)
    assert np.abs((np.eye(C) + A) @ T - np.diag(beta)).max() < 1e-12
    assert np.abs(np.triu(T, 1)).max() == 0.0
    assert np.allclose(np.diag(T), beta)


# ---- gated (Gated DeltaNet) oracle ------------------------------------------

from oracle import gated_delta_rule_decode_step, gated_delta_rule_forward  # noqa: E402
from pins_gated import ALL_GATED_PINS  # noqa: E402


@pytest.mark.parametrize("pin", ALL_GATED_PINS, ids=lambda p: p.__name__)
def test_gated_oracle_pin(pin):
    rng = np.random.default_rng(4321)
    err = pin(gated_delta_rule_forward, rng)
    assert err < PIN_TOL, f"{pin.__name__}: max deviation {err:.3e}"


def test_gated_decode_step_is_forward_at_one_token():
    rng = np.random.default_rng(17)
    B, H, L, dk, dv = 2, 3, 7, 6, 4
    q, k = rng.standard_normal((B, H, L, dk)), rng.standard_normal((B, H, L, dk))
    v = rng.standard_normal((B, H, L, dv))
    alpha, beta = rng.uniform(0, 1, (B, H, L)), rng.uniform(0, 1, (B, H, L))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.1
    o_ref, S_ref = gated_delta_rule_forward(q, k, v, alpha, beta, S0)
    S = S0
    for t in range(L):
        o_t, S = gated_delta_rule_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], alpha[:, :, t],
                                              beta[:, :, t], S)
        assert np.abs(o_t - o_ref[:, :, t]).max() < 1e-12
    assert np.abs(S - S_ref).max() < 1e-12


def test_gated_decode_step_identity():
    """o = q S_new = alpha q S + (q . k) u with u = beta (v - alpha k S): the
    single-read form the gated decode kernel uses."""
    rng = np.random.default_rng(18)
    B, H, dk, dv = 2, 2, 5, 3
    q, k = rng.standard_normal((B, H, dk)), rng.standard_normal((B, H, dk))
    v = rng.standard_normal((B, H, dv))
    alpha, beta = rng.uniform(0, 1, (B, H)), rng.uniform(0, 1, (B, H))
    S = rng.standard_normal((B, H, dk, dv))
    o, S_new = gated_delta_rule_decode_step(q, k, v, alpha, beta, S)
    r = np.einsum("bhk,bhkv->bhv", k, S)
    p = np.einsum("bhk,bhkv->bhv", q, S)
    u = beta[..., None] * (v - alpha[..., None] * r)
    o2 = alpha[..., None] * p + np.einsum("bhk,bhk->bh", q, k)[..., None] * u
    assert np.abs(o - o2).max() < 1e-12
    S2 = alpha[..., None, None] * S + k[..., :, None] * u[..., None, :]
    assert np.abs(S_new - S2).max() < 1e-12


@pytest.mark.parametrize("C,SB", [(1, None), (7, None), (16, None), (64, None), (64, 32), (128, 32)])
@pytest.mark.parametrize("L", [150, 64])
def test_gated_chunked_form_equals_recurrence(C, SB, L):
    from wy_model import gated_chunked_forward
    rng = np.random.default_rng(C * 100 + L)
    q, k, v, beta, S0 = _rand_head(rng, L, 16, 12)
    alpha = rng.uniform(0.5, 1.0, L)
    alpha[::13] = 1.0
    alpha[5] = 0.0                       # one memory wipe
    o_ref, S_ref = gated_delta_rule_forward(q[None, None], k[None, None], v[None, None],
                                            alpha[None, None], beta[None, None], S0[None, None])
    o, S = gated_chunked_forward(q, k, v, alpha, beta, S0, C, SB)
    assert np.abs(o - o_ref[0, 0]).max() < 1e-10
    assert np.abs(S - S_ref[0, 0]).max() < 1e-10
