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


def worst_head(got, ref) -> tuple:
    """(b, h) of the head with the largest max |err|, and that head's
    max|err| / RMS(ref) over the whole tensor (the per-head worst)."""
    g, r = to64(got), to64(ref)
    rms = np.sqrt(np.mean(r * r))
    per = np.abs(g - r).reshape(g.shape[0], g.shape[1], -1).max(axis=-1)
    b, h = np.unravel_index(int(np.argmax(per)), per.shape)
    return (int(b), int(h)), float(per[b, h] / (rms if rms > 0 else 1.0))


def record(test: str, **values) -> None:
    """Appends one JSON line of measured errors to the file named by the
    DN_PARITY_LOG environment variable (nothing when it is unset)."""
    import json
    import os

    path = os.environ.get("DN_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps({"test": test, **values}) + "\n")


def check_bf16_out(o16, o32, ref, e32: float) -> tuple:
    """o stored in bf16 is the fp32 result rounded to nearest: within one bf16
    step (2^-8 relative) of the fp32 output everywhere, so its error against
    the oracle is at most the fp32 output's error plus that rounding.
    Returns (max|err|/RMS(ref) of the bf16 output, the same for the oracle's
    own values rounded to bf16 -- the floor no bf16 output can go below)."""
    g16 = to64(o16)
    g32 = to64(o32)
    r = to64(ref)
    assert np.all(np.abs(g16 - g32) <= 2.0 ** -8 * np.abs(g32)), \
        "bf16 output is not a rounding of the fp32 output"
    rms = np.sqrt(np.mean(r * r))
    e16 = float(np.abs(g16 - r).max() / rms)
    bound = e32 + 2.0 ** -8 * float(np.abs(g32).max()) / rms
    assert e16 <= bound, f"bf16 output error {e16:.3e} above fp32 error + rounding {bound:.3e}"
    floor = float(np.abs(to64(torch.from_numpy(r).to(torch.bfloat16)) - r).max() / rms)
    return e16, floor
