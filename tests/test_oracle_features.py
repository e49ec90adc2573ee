"""Pins for the oracle's feature maps (oracle/features.py) and planted
mistakes that each of them must catch.

The maps are the layer's q, k = normalise(silu(.)) and beta = sigmoid(logit)
(page "GPT-2 から Kimi K3 まで、AI モデルの進化を解説", section "DeltaNet (Fast
weight programmers)").  Each pin checks the oracle against something other
than itself: values with closed forms, identities of silu and sigmoid, the
unit norm and sign of every normalised row, PyTorch's documented eps branch,
exact bf16 ties, and a row worked by hand.
"""

import math

import numpy as np
import pytest
import torch

from oracle import feature_maps, l2_normalize, round_to_bf16, sigmoid, silu

LN3 = math.log(3.0)
# Hand-worked row: x = [0, ln 3, -ln 3, 0].  sigmoid(ln 3) = 1/(1 + 1/3) = 3/4
# and sigmoid(-ln 3) = 1/4, so silu(x) = ln 3 [0, 3/4, -1/4, 0], whose norm is
# ln 3 sqrt(5/8); the normalised row is [0, 3/4, -1/4, 0] / sqrt(5/8)
# = [0, 0.75 sqrt(1.6), -0.25 sqrt(1.6), 0].
HAND_X = [0.0, LN3, -LN3, 0.0]
HAND_F64 = [0.0, 0.75 * math.sqrt(1.6), -0.25 * math.sqrt(1.6), 0.0]
# Its bf16 rounding, by hand: 0.94868... = 242.86/256 -> 243/256; -0.31623... =
# -0.5 * 161.91/256 -> -0.5 * 162/256.
HAND_BF16 = [0.0, 243 / 256, -81 / 256, 0.0]


# --- the scalar maps ------------------------------------------------------

def test_sigmoid_closed_forms():
    assert sigmoid(0.0) == 0.5
    assert abs(sigmoid(LN3) - 0.75) < 1e-15
    assert abs(sigmoid(-LN3) - 0.25) < 1e-15
    assert sigmoid(-800.0) == 0.0 and sigmoid(800.0) == 1.0  # no overflow NaN
    x = np.random.default_rng(0).standard_normal(1000) * 5
    assert np.max(np.abs(sigmoid(x) + sigmoid(-x) - 1.0)) < 1e-15


def test_silu_closed_forms():
    assert silu(0.0) == 0.0
    assert abs(silu(1.0) - math.e / (1.0 + math.e)) < 1e-15
    assert abs(silu(LN3) - 0.75 * LN3) < 1e-15
    assert abs(silu(40.0) - 40.0) < 1e-12
    assert silu(-800.0) == 0.0  # -800 e^-800 underflows, no NaN
    # silu(-x) = -x sigmoid(-x) = -x (1 - sigmoid(x)) = silu(x) - x
    x = np.random.default_rng(1).standard_normal(1000) * 4
    assert np.max(np.abs(silu(-x) - (silu(x) - x))) < 1e-14


def test_l2_normalize_rows():
    assert np.allclose(l2_normalize(np.array([3.0, 4.0])), [0.6, 0.8], rtol=0, atol=1e-16)
    x = np.random.default_rng(2).standard_normal((2, 3, 5, 16))
    y = l2_normalize(x)
    assert np.max(np.abs(np.linalg.norm(y, axis=-1) - 1.0)) < 1e-15
    assert np.all(np.sign(y) == np.sign(x))
    # eps branch (PyTorch's F.normalize: x / max(||x||, 1e-12))
    assert np.all(l2_normalize(np.zeros((2, 8))) == 0.0)
    tiny = np.full(4, 1e-14)  # norm 2e-14 < eps
    assert np.allclose(l2_normalize(tiny), tiny / 1e-12, rtol=1e-15, atol=0)


def test_round_to_bf16_ties_and_library_agreement():
    one_ulp = 2.0 ** -7  # bf16 spacing on [1, 2)
    cases = {1 + 2 ** -8: 1.0,                      # tie, even neighbour is 1
             1 + 3 * 2 ** -8: 1 + 2 * one_ulp,      # tie, even neighbour above
             -(1 + 2 ** -8): -1.0,
             1 + 2 ** -8 + 2 ** -40: 1 + one_ulp,   # just past the tie
             1 + 2 ** -8 - 2 ** -40: 1.0,
             0.5 + 2 ** -9 + 2 ** -30: 0.5 + 2 ** -8,
             1.3 * 2 ** -130: 10 * 2 ** -133}       # subnormal spacing 2^-133
    for x, want in cases.items():
        assert round_to_bf16(np.array(x)) == want, x
    # On fp32-representable values it must agree with PyTorch's fp32 -> bf16.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 3, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), ref)


# --- pins on the composite map (also run against the planted mistakes) ----

def pin_hand_row(fm):
    x = np.array([HAND_X, HAND_X[::-1]])
    qh, kh, b = fm(x, x, np.array([0.0, LN3, -LN3]), "f64")
    want = np.array([HAND_F64, HAND_F64[::-1]])
    return max(np.max(np.abs(qh - want)), np.max(np.abs(kh - want)),
               np.max(np.abs(b - [0.5, 0.75, 0.25])))


def pin_hand_row_bf16(fm):
    x = np.array([HAND_X])
    qh, kh, _ = fm(x, x, np.zeros(1), "bf16")
    return max(np.max(np.abs(qh - [HAND_BF16])), np.max(np.abs(kh - [HAND_BF16])))


def pin_unit_rows_and_sign(fm):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 3, 5, 16)) * 2
    k = rng.standard_normal((2, 3, 5, 16)) * 0.5
    qh, kh, _ = fm(q, k, np.zeros((2, 3, 5)), "f64")
    err = 0.0
    for x, y in ((q, qh), (k, kh)):
        err = max(err, np.max(np.abs(np.linalg.norm(y, axis=-1) - 1.0)))
        if not np.all(np.sign(y) == np.sign(x)):  # silu keeps the sign
            err = np.inf
    return err


def pin_zero_and_tiny_rows(fm):
    x = np.zeros((3, 8))
    x[1] = -1e-13  # silu ~ x / 2: norm ~1.4e-13 < eps
    x[2, 0] = 1.0
    qh, kh, _ = fm(x, x, np.zeros(3), "f64")
    want1 = (x[1] / (1 + np.exp(-x[1]))) / 1e-12
    err = max(np.max(np.abs(qh[0])), np.max(np.abs(qh[1] - want1)) / np.max(np.abs(want1)),
              np.max(np.abs(qh[2] - np.eye(8)[0])))
    return np.inf if not np.all(np.isfinite(qh)) else err


def pin_large_inputs(fm):
    x = np.array([[40.0, -40.0, 0.0, 0.0], [-800.0, 800.0, 1.0, 0.0]])
    qh, kh, b = fm(x, x, np.array([-800.0, 800.0]), "f64")
    if not (np.all(np.isfinite(qh)) and np.all(np.isfinite(b))):
        return np.inf
    s1 = math.e / (1 + math.e)  # silu(1)
    n = math.hypot(800.0, s1)
    want = np.array([[1.0, 0, 0, 0], [0, 800.0 / n, s1 / n, 0]])
    return max(np.max(np.abs(qh - want)), np.max(np.abs(b - [0.0, 1.0])))


FEATURE_PINS = [pin_hand_row, pin_hand_row_bf16, pin_unit_rows_and_sign, pin_zero_and_tiny_rows,
                pin_large_inputs]
FEATURE_TOL = 1e-14


@pytest.mark.parametrize("pin", FEATURE_PINS, ids=lambda p: p.__name__)
def test_oracle_feature_pin(pin):
    assert pin(feature_maps) < FEATURE_TOL


# --- planted mistakes (copies of the maps on the CPU) ---------------------

def _mutant_maps(mutant):
    def sig(x):
        x = np.asarray(x, float)
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(x if mutant == "sigmoid_flipped" else -x))

    def act(x):
        x = np.asarray(x, float)
        if mutant == "no_silu":
            return x
        if mutant == "relu":
            return np.maximum(x, 0.0)
        if mutant == "elu_plus_one":  # linear attention's map, not this layer's
            return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
        return x * sig(x) if mutant != "sigmoid_flipped" else x / (1.0 + np.exp(-x))

    def norm(x):
        axis = -2 if mutant == "wrong_axis" else -1
        if mutant == "l1_norm":
            n = np.sum(np.abs(x), axis=axis, keepdims=True)
        else:
            n = np.sqrt(np.sum(x * x, axis=axis, keepdims=True))
        if mutant == "no_eps":
            with np.errstate(invalid="ignore", divide="ignore"):
                return x / n
        return x / np.maximum(n, 1e-12)

    def fm(q, k, bl, store):
        if mutant == "normalize_then_silu":
            qh, kh = act(norm(np.asarray(q, float))), act(norm(np.asarray(k, float)))
        else:
            qh, kh = norm(act(q)), norm(act(k))
        b = np.asarray(bl, float) if mutant == "beta_not_squashed" else sig(bl)
        if store == "bf16":
            if mutant == "truncate_bf16":
                m, e = np.frexp(qh)
                qh = np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)
                m, e = np.frexp(kh)
                kh = np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)
            else:
                qh, kh = round_to_bf16(qh), round_to_bf16(kh)
        return qh, kh, b

    return fm


FEATURE_MUTANTS = ["no_silu", "relu", "elu_plus_one", "wrong_axis", "l1_norm", "no_eps",
                   "sigmoid_flipped", "beta_not_squashed", "normalize_then_silu", "truncate_bf16"]


def test_unmutated_feature_copy_passes_every_pin():
    for pin in FEATURE_PINS:
        assert pin(_mutant_maps(None)) < FEATURE_TOL, pin.__name__


@pytest.mark.parametrize("mutant", FEATURE_MUTANTS)
def test_feature_mutant_is_caught(mutant):
    caught = []
    for pin in FEATURE_PINS:
        try:
            err = pin(_mutant_maps(mutant))
        except (ValueError, IndexError, FloatingPointError):
            err = np.inf
        if not err < FEATURE_TOL:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant!r} passed every pin"


def test_feature_maps_then_core_matches_direct_core():
    """The composite (maps, then the fp64 recurrence) is the core run on the
    mapped operands: nothing else is added between the two."""
    from oracle import delta_rule_forward

    rng = np.random.default_rng(6)
    q, k = rng.standard_normal((2, 1, 2, 9, 8))
    v = rng.standard_normal((1, 2, 9, 8))
    bl = rng.standard_normal((1, 2, 9))
    qh, kh, b = feature_maps(q, k, bl, "f64")
    o, S = delta_rule_forward(qh, kh, v, b, None)
    assert np.all(np.isfinite(o)) and o.shape == v.shape
    # unit keys and beta in (0, 1): the transition I - beta k^T k is a
    # contraction, so the state norm is bounded by the sum of the writes.
    bound = np.sum(b[..., None] * np.linalg.norm(v, axis=-1)[..., None], axis=2)
    assert np.all(np.linalg.norm(S, axis=(-2, -1)) <= 2 * bound[..., 0] + 1e-12)
