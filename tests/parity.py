"""Parity bars between the HIP path and the fp64 oracle.

* fp32 inputs: max_i |g_i - r_i| / max_i |r_i| <= 1e-4, per output tensor.
  (A max relative error taken element by element is ill-posed where the
  reference passes through zero; the bar is relative to the tensor's scale.)
* bf16 inputs: max_i |g_i - r_i| <= 2e-2 * RMS(r), per output tensor, with the
  oracle run on the same bf16-rounded inputs upcast exactly to fp64.
"""

from __future__ import annotations

import numpy as np
import torch

F32_REL_TOL = 1e-4
BF16_RMS_TOL = 2e-2


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def err_f32(got, ref) -> float:
    g, r = to64(got), to64(ref)
    scale = np.abs(r).max()
    return float(np.abs(g - r).max() / (scale if scale > 0 else 1.0))


def err_bf16(got, ref) -> float:
    g, r = to64(got), to64(ref)
    rms = np.sqrt(np.mean(r * r))
    return float(np.abs(g - r).max() / (rms if rms > 0 else 1.0))


def assert_parity(got, ref, in_dtype: str, what: str):
    """Asserts the bar for ``in_dtype`` ("f32" or "bf16") and returns the error."""
    if in_dtype == "f32":
        e = err_f32(got, ref)
        assert e <= F32_REL_TOL, f"{what}: max|err|/max|ref| = {e:.3e} > {F32_REL_TOL}"
    else:
        e = err_bf16(got, ref)
        assert e <= BF16_RMS_TOL, f"{what}: max|err|/RMS(ref) = {e:.3e} > {BF16_RMS_TOL}"
    return e
