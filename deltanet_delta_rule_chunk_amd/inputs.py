"""Seeded synthetic inputs for the delta-rule forward and decode step.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It holds only the input recipe (random draws, the per-token L2
normalisation of the keys, the sigmoid that turns a logit into a write
strength, and the casts to the storage dtype); none of the recurrence's
arithmetic lives here.

Recipe (identical for every workload):
  * ``rng = numpy.random.default_rng(seed)`` (PCG64), fp64 draws in the fixed
    order q, k, v (each ``[B,H,L,d]`` standard normal, C order), then the
    beta logits ``[B,H,L]``, then (only where the workload has one) the
    initial state ``[B,H,d_k,d_v]`` with standard deviation 0.1 (variance
    0.01).
  * k <- k / max(||k||_2, 1e-12) per token, in fp64, before the cast.
  * beta = 1 / (1 + exp(-logit)); on workloads with "overwrite heads", heads
    h < n_overwrite_heads get beta = 1 exactly.
  * q, k, v are cast to the workload's storage dtype (bf16 with
    round-to-nearest-even, or fp32); beta and the state are cast to fp32.

Draws for a large tensor are made one (b,h) slice at a time; PCG64's
standard-normal stream is the same whether a block is drawn at once or in
consecutive pieces, so the values equal one big draw while the peak host
memory stays at one slice of fp64.

Decode steps: the state is drawn from ``default_rng(seed)``; step s draws its
q, k, v, beta-logit from ``default_rng([seed, s + 1])`` with the same
transforms, so any step can be made on its own.

Gated form (Gated DeltaNet): the decay alpha comes from a stream of its own,
``default_rng([seed, 7])`` for a chunked forward (``[B,H,L]`` in C order) and
``default_rng([seed, s + 1, 7])`` for decode step s (``[B,H]``), as
alpha = sigmoid(N(3, 1)) in fp64 then cast to fp32 (a decay
per token on average 0.93, from ~0.25 to ~0.9996), so the draws of the
other inputs are the same with or without the gate.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class ChunkWorkload:
    """One chunked-forward workload: shapes, chunk size, dtype, state recipe."""

    name: str
    B: int
    H: int
    L: int
    d_k: int
    d_v: int
    C: int
    dtype: str  # "f32" or "bf16": storage dtype of q, k, v
    s0_std: Optional[float] = None  # None: the forward starts from the zero state
    n_overwrite_heads: int = 0  # heads h < this get beta == 1 exactly

    @property
    def tokens(self) -> int:
        return self.B * self.L


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """The single-token decode workload: B sequences x H heads, fp32 state."""

    name: str
    B: int
    H: int
    d_k: int
    d_v: int
    steps: int
    dtype: str
    s_std: float


# The five workloads the method is exercised and measured on.  Index 0 is the
# small fp32 case the oracle finishes in well under a second; 3 is the
# long-context case; 4 is the decode step.
WORKLOADS = [
    ChunkWorkload("fp32_B1_H2_L256_d64_C64", 1, 2, 256, 64, 64, 64, "f32"),
    ChunkWorkload("bf16_B4_H12_L2048_d64_C64", 4, 12, 2048, 64, 64, 64, "bf16"),
    ChunkWorkload("bf16_B2_H16_L8192_d128_C64_S0_overwrite", 2, 16, 8192, 128, 128, 64, "bf16",
                  s0_std=0.1, n_overwrite_heads=8),
    ChunkWorkload("bf16_B1_H32_L65536_d128_C128", 1, 32, 65536, 128, 128, 128, "bf16"),
    DecodeWorkload("decode_bf16_B256_H32_d128", 256, 32, 128, 128, 1000, "bf16", 0.1),
]

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _draw_normal(rng: np.random.Generator, shape, cast) -> torch.Tensor:
    """Standard-normal draw of ``shape`` (C order), slice by slice over the
    leading two axes, each slice passed through ``cast`` (fp64 numpy ->
    torch tensor).  Returns the concatenated torch tensor."""
    lead = shape[0] * shape[1]
    tail = tuple(shape[2:])
    out = None
    for i in range(lead):
        piece = cast(rng.standard_normal(tail))
        if out is None:
            out = torch.empty((lead,) + tuple(piece.shape), dtype=piece.dtype)
        out[i] = piece
    return out.reshape(tuple(shape[:2]) + tuple(out.shape[1:]))


def _to_storage(dtype: torch.dtype):
    def cast(a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(a).to(dtype)
    return cast


def _unit_rows_to_storage(dtype: torch.dtype):
    def cast(a: np.ndarray) -> torch.Tensor:
        n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True))
        return torch.from_numpy(a / np.maximum(n, 1e-12)).to(dtype)
    return cast


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def make_chunk_inputs(w: ChunkWorkload, seed: int = 0, L: Optional[int] = None) -> dict:
    """Host (CPU) torch tensors for one chunked-forward call.

    Returns dict(q, k, v, beta, S0) with q,k ``[B,H,L,d_k]``, v ``[B,H,L,d_v]``
    in the workload's storage dtype, beta ``[B,H,L]`` fp32 and S0
    ``[B,H,d_k,d_v]`` fp32 or None.  ``L`` overrides the workload's length
    (used for ragged-tail cases)."""
    L = w.L if L is None else L
    dt = _TORCH_DTYPE[w.dtype]
    rng = np.random.default_rng(seed)
    q = _draw_normal(rng, (w.B, w.H, L, w.d_k), _to_storage(dt))
    k = _draw_normal(rng, (w.B, w.H, L, w.d_k), _unit_rows_to_storage(dt))
    v = _draw_normal(rng, (w.B, w.H, L, w.d_v), _to_storage(dt))
    logit = rng.standard_normal((w.B, w.H, L))
    beta = _sigmoid(logit)
    if w.n_overwrite_heads:
        beta[:, : w.n_overwrite_heads, :] = 1.0
    beta = torch.from_numpy(beta).to(torch.float32)
    S0 = None
    if w.s0_std is not None:
        S0 = _draw_normal(rng, (w.B, w.H, w.d_k, w.d_v),
                          lambda a: torch.from_numpy(a * w.s0_std).to(torch.float32))
    return dict(q=q, k=k, v=v, beta=beta, S0=S0)


def _alpha_from(rng: np.random.Generator, shape) -> torch.Tensor:
    return torch.from_numpy(_sigmoid(3.0 + rng.standard_normal(shape))).to(torch.float32)


def make_chunk_alpha(w: ChunkWorkload, seed: int = 0, L: Optional[int] = None) -> torch.Tensor:
    """Per-token decay ``[B,H,L]`` fp32 of the gated forward."""
    L = w.L if L is None else L
    return _alpha_from(np.random.default_rng([seed, 7]), (w.B, w.H, L))


def make_decode_alpha(w: DecodeWorkload, step: int, seed: int = 0) -> torch.Tensor:
    """Per-(b, h) decay ``[B,H]`` fp32 of gated decode step ``step``."""
    return _alpha_from(np.random.default_rng([seed, step + 1, 7]), (w.B, w.H))


def make_chunk_kda_alpha(w: ChunkWorkload, seed: int = 0, L: Optional[int] = None) -> torch.Tensor:
    """Per-token, per-key-dimension decay ``[B,H,L,d_k]`` fp32 of the KDA
    forward: sigmoid(N(3, 1)) per element, from ``default_rng([seed, 13])``."""
    L = w.L if L is None else L
    return _alpha_from(np.random.default_rng([seed, 13]), (w.B, w.H, L, w.d_k))


def make_decode_kda_alpha(w: DecodeWorkload, step: int, seed: int = 0) -> torch.Tensor:
    """Per-key-dimension decay ``[B,H,d_k]`` fp32 of KDA decode step ``step``."""
    return _alpha_from(np.random.default_rng([seed, step + 1, 13]), (w.B, w.H, w.d_k))


def make_decode_state(w: DecodeWorkload, seed: int = 0) -> torch.Tensor:
    """Initial decode state ``[B,H,d_k,d_v]`` fp32, std ``w.s_std``."""
    rng = np.random.default_rng(seed)
    return _draw_normal(rng, (w.B, w.H, w.d_k, w.d_v),
                        lambda a: torch.from_numpy(a * w.s_std).to(torch.float32))


def make_decode_step_inputs(w: DecodeWorkload, step: int, seed: int = 0) -> dict:
    """Inputs of decode step ``step``: q,k ``[B,H,d_k]``, v ``[B,H,d_v]`` in the
    storage dtype, beta ``[B,H]`` fp32."""
    dt = _TORCH_DTYPE[w.dtype]
    rng = np.random.default_rng([seed, step + 1])
    q = torch.from_numpy(rng.standard_normal((w.B, w.H, w.d_k))).to(dt)
    kk = rng.standard_normal((w.B, w.H, w.d_k))
    kk = kk / np.maximum(np.sqrt(np.sum(kk * kk, axis=-1, keepdims=True)), 1e-12)
    k = torch.from_numpy(kk).to(dt)
    v = torch.from_numpy(rng.standard_normal((w.B, w.H, w.d_v))).to(dt)
    beta = torch.from_numpy(_sigmoid(rng.standard_normal((w.B, w.H)))).to(torch.float32)
    return dict(q=q, k=k, v=v, beta=beta)


def make_chunk_raw_inputs(w: ChunkWorkload, seed: int = 0, L: Optional[int] = None) -> dict:
    """Host tensors for a chunked forward fed by the layer's raw projections
    (the feature maps run first): dict(q_raw, k_raw, v, beta_logit, S0) with
    q_raw, k_raw ``[B,H,L,d_k]`` and v ``[B,H,L,d_v]`` standard normal in the
    storage dtype (a projection's output), beta_logit ``[B,H,L]`` standard
    normal fp32, S0 as in ``make_chunk_inputs``.  Its own stream,
    ``default_rng([seed, 11])``, draws in that order."""
    L = w.L if L is None else L
    dt = _TORCH_DTYPE[w.dtype]
    rng = np.random.default_rng([seed, 11])
    q = _draw_normal(rng, (w.B, w.H, L, w.d_k), _to_storage(dt))
    k = _draw_normal(rng, (w.B, w.H, L, w.d_k), _to_storage(dt))
    v = _draw_normal(rng, (w.B, w.H, L, w.d_v), _to_storage(dt))
    logit = torch.from_numpy(rng.standard_normal((w.B, w.H, L))).to(torch.float32)
    S0 = None
    if w.s0_std is not None:
        S0 = _draw_normal(rng, (w.B, w.H, w.d_k, w.d_v),
                          lambda a: torch.from_numpy(a * w.s0_std).to(torch.float32))
    return dict(q_raw=q, k_raw=k, v=v, beta_logit=logit, S0=S0)


def make_decode_raw_step_inputs(w: DecodeWorkload, step: int, seed: int = 0) -> dict:
    """Raw inputs of decode step ``step`` (the feature maps run in the step):
    q_raw, k_raw ``[B,H,d_k]``, v ``[B,H,d_v]`` standard normal in the
    storage dtype, beta_logit ``[B,H]`` standard normal fp32, from
    ``default_rng([seed, step + 1, 11])``."""
    dt = _TORCH_DTYPE[w.dtype]
    rng = np.random.default_rng([seed, step + 1, 11])
    q = torch.from_numpy(rng.standard_normal((w.B, w.H, w.d_k))).to(dt)
    k = torch.from_numpy(rng.standard_normal((w.B, w.H, w.d_k))).to(dt)
    v = torch.from_numpy(rng.standard_normal((w.B, w.H, w.d_v))).to(dt)
    logit = torch.from_numpy(rng.standard_normal((w.B, w.H))).to(torch.float32)
    return dict(q_raw=q, k_raw=k, v=v, beta_logit=logit)


def scaled_chunk_workload(w: ChunkWorkload, **changes) -> ChunkWorkload:
    """A copy of ``w`` with some fields changed (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact upcast of a stored tensor (bf16/fp32) to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
