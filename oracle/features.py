"""fp64 CPU oracle for the DeltaNet layer's feature maps.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path.

What it computes.  The layer forward on the page "GPT-2 から Kimi K3 まで、AI
モデルの進化を解説" (news.ainew.jp), section "DeltaNet (Fast weight
programmers)", prepares the core's operands from the projections before the
delta rule runs:
    q <- L2-normalise(silu(q)),   k <- L2-normalise(silu(k))   along the head
    dimension, and the write strength beta = sigmoid(w_beta x).
This module writes those three maps out from their definitions:
    silu(x)    = x * sigmoid(x) = x / (1 + e^{-x})
    sigmoid(x) = 1 / (1 + e^{-x})
    normalise(x) = x / max(||x||_2, eps),  eps = 1e-12
(the page calls PyTorch's F.normalize with its default p = 2 and eps = 1e-12).
The beta projection w_beta x is a learned weight and stays outside: the input
here is its output, the per-(batch, head, token) logit.

Readings taken where the page is silent (each listed in the design notes):
the maps are evaluated exactly (fp64 here) and their q and k outputs are then
held in the dtype the core takes (for bf16 inputs: rounded to the nearest
bf16, ties to even), as a bf16 model holds them; beta stays fp32 (rounded to
the nearest fp32 here).

Pins (tests/test_oracle_features.py): silu and sigmoid at values with closed
forms (0, 1, log 3, large |x|) and their reflection identities; unit norm and
direction of every normalised row; the eps branch at zero and tiny rows; the
bf16 rounding at exact ties; a hand-worked row; and planted mistakes (a
dropped silu, the wrong normalisation axis, a missing eps, a flipped sigmoid,
rounding by truncation) that each fail one of those pins.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

NORMALIZE_EPS = 1e-12


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + e^{-x}) in fp64 (the page's torch.sigmoid on the beta logits)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) in fp64 (the page's F.silu on q and k)."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def l2_normalize(x: np.ndarray, eps: float = NORMALIZE_EPS) -> np.ndarray:
    """x / max(||x||_2, eps) along the last (head) dimension (F.normalize, p = 2)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to
    even, returned as fp64.  Direct from fp64: frexp gives x = m 2^e with
    0.5 <= |m| < 1, so m 2^8 holds the kept bits left of the point and rint
    (round half to even) rounds it exactly.  Below bf16's smallest normal
    (2^-126) the spacing stays 2^-133 (subnormals).  Magnitudes past bf16's
    range are not expected here (the maps' outputs lie in [-1, 1])."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    m = np.ldexp(x, -e)  # = m unless x is below the normal range
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def feature_maps(q_raw: np.ndarray, k_raw: np.ndarray, beta_logit: np.ndarray,
                 store: str = "bf16") -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The core's operands from the raw projections.

    q_raw, k_raw: [..., d_k]; beta_logit: [...].  ``store`` is the dtype the
    core takes q and k in: "bf16" rounds the exact maps to bf16, "f32" to
    fp32, "f64" keeps them exact.  beta is rounded to fp32 unless store is
    "f64".  Returns fp64 arrays (q_hat, k_hat, beta)."""
    qh = l2_normalize(silu(q_raw))
    kh = l2_normalize(silu(k_raw))
    b = sigmoid(beta_logit)
    if store == "bf16":
        qh, kh = round_to_bf16(qh), round_to_bf16(kh)
    elif store == "f32":
        qh, kh = (x.astype(np.float32).astype(np.float64) for x in (qh, kh))
    elif store != "f64":
        raise ValueError(f"store must be bf16, f32 or f64 (got {store!r})")
    if store != "f64":
        b = b.astype(np.float32).astype(np.float64)
    return qh, kh, b
