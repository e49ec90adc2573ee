"""Plant plausible mistakes in copies of the recurrence (on the CPU) and show
that each one trips at least one pin.  This is what makes the pins worth
trusting: a pin set that a wrong oracle could pass would pin nothing."""

import numpy as np
import pytest

from pins import ALL_PINS, PIN_TOL


def _loop(q, k, v, beta, S0, mutant):
    q, k, v, beta = (np.asarray(x, float) for x in (q, k, v, beta))
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.asarray(S0, float).copy()
    if mutant == "ignore_S0":
        S = np.zeros((B, H, dk, dv))
    o = np.empty((B, H, L, dv))
    for t in range(L):
        kt = k[:, :, t, None, :]
        if mutant == "previous_key" and t > 0:
            kt = k[:, :, t - 1, None, :]
        if mutant == "transposed_read":
            v_old = (S @ np.swapaxes(kt, -1, -2)).swapaxes(-1, -2)
        else:
            v_old = kt @ S
        b = beta[:, :, t, None, None]
        vt = v[:, :, t, None, :]
        if mutant == "sign_flip":
            u = b * (vt + v_old)
        elif mutant == "beta_on_v_only":
            u = b * vt - v_old
        elif mutant == "no_beta":
            u = vt - v_old
        elif mutant == "beta_twice":
            u = b * b * (vt - v_old)
        else:
            u = b * (vt - v_old)
        o_before = (q[:, :, t, None, :] @ S)[:, :, 0, :]
        if mutant == "write_at_query":
            S = S + np.swapaxes(q[:, :, t, None, :], -1, -2) @ u
        elif mutant == "no_erase":
            S = S + np.swapaxes(kt, -1, -2) @ (b * vt)
        else:
            S = S + np.swapaxes(kt, -1, -2) @ u
        if mutant == "read_before_write":
            o[:, :, t, :] = o_before
        elif mutant == "read_with_key":
            o[:, :, t, :] = (kt @ S)[:, :, 0, :]
        else:
            o[:, :, t, :] = (q[:, :, t, None, :] @ S)[:, :, 0, :]
    if mutant == "state_not_returned":
        return o, np.zeros_like(S)
    return o, S


MUTANTS = ["ignore_S0", "previous_key", "transposed_read", "sign_flip", "beta_on_v_only",
           "no_beta", "beta_twice", "write_at_query", "no_erase", "read_before_write",
           "read_with_key", "state_not_returned"]


def test_unmutated_copy_passes_every_pin():
    for pin in ALL_PINS:
        err = pin(lambda *a: _loop(*a, mutant=None), np.random.default_rng(5))
        assert err < PIN_TOL, pin.__name__


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(mutant):
    caught = []
    for pin in ALL_PINS:
        try:
            err = pin(lambda *a: _loop(*a, mutant=mutant), np.random.default_rng(5))
        except (ValueError, IndexError):
            err = np.inf  # a shape error is also a failed pin
        if not err < PIN_TOL:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant!r} passed every pin"


# ---- gated recurrence ---------------------------------------------------------

from pins_gated import ALL_GATED_PINS  # noqa: E402


def _gated_loop(q, k, v, alpha, beta, S0, mutant):
    q, k, v, alpha, beta = (np.asarray(x, float) for x in (q, k, v, alpha, beta))
    B, H, L, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.asarray(S0, float).copy()
    o = np.empty((B, H, L, dv))
    for t in range(L):
        a = alpha[:, :, t, None, None]
        if mutant == "previous_alpha" and t > 0:
            a = alpha[:, :, t - 1, None, None]
        kt = k[:, :, t, None, :]
        b = beta[:, :, t, None, None]
        vt = v[:, :, t, None, :]
        if mutant == "decay_after_write":
            S = S + np.swapaxes(kt, -1, -2) @ (b * (vt - kt @ S))
            S = a * S
        elif mutant == "delta_reads_undecayed":
            u = b * (vt - kt @ S)
            S = a * S + np.swapaxes(kt, -1, -2) @ u
        elif mutant == "decay_write_too":
            S = a * S
            S = S + a * (np.swapaxes(kt, -1, -2) @ (b * (vt - kt @ S)))
        elif mutant == "no_decay_of_S0" and t == 0:
            S = S + np.swapaxes(kt, -1, -2) @ (b * (vt - kt @ S))
        else:
            S = a * S
            S = S + np.swapaxes(kt, -1, -2) @ (b * (vt - kt @ S))
        if mutant == "decay_on_read_only":
            o[:, :, t, :] = (q[:, :, t, None, :] @ (a * S))[:, :, 0, :]
        else:
            o[:, :, t, :] = (q[:, :, t, None, :] @ S)[:, :, 0, :]
    return o, S


GATED_MUTANTS = ["previous_alpha", "decay_after_write", "delta_reads_undecayed", "decay_write_too",
                 "no_decay_of_S0", "decay_on_read_only"]


def test_unmutated_gated_copy_passes_every_pin():
    for pin in ALL_GATED_PINS:
        err = pin(lambda *a: _gated_loop(*a, mutant=None), np.random.default_rng(6))
        assert err < PIN_TOL, pin.__name__


@pytest.mark.parametrize("mutant", GATED_MUTANTS)
def test_gated_mutant_is_caught(mutant):
    caught = []
    for pin in ALL_GATED_PINS:
        try:
            err = pin(lambda *a: _gated_loop(*a, mutant=mutant), np.random.default_rng(6))
        except (ValueError, IndexError):
            err = np.inf
        if not err < PIN_TOL:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant!r} passed every pin"
