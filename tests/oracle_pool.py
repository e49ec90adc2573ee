"""The fp64 oracle over many heads at once, in parallel worker processes.

Every form of the recurrence (plain, gated, per-dimension decay, with feature
maps) treats each (batch, head) pair on its own: the oracle on a group of
heads is the oracle on the whole tensor restricted to those heads.  This
module only splits the head axis into groups, runs the unchanged oracle
functions on each group in a separate process (``spawn`` start method, so the
workers never inherit the GPU state of the test process) and puts the results
back in place.  It adds no arithmetic of its own.

Worker count: the CPUs this process may run on, at most 16 (the host share of
one GPU), and never more than the number of heads.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
from typing import Callable, Optional, Sequence

import numpy as np


def n_workers(n_heads: int) -> int:
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        cpus = os.cpu_count() or 1
    return max(1, min(16, cpus, n_heads))


def _host(a) -> Optional[np.ndarray]:
    """A CPU numpy view of a tensor or array, in a dtype that holds its values
    exactly (bf16 -> fp32), flattened over (B, H) to one head axis."""
    if a is None:
        return None
    try:
        import torch

        if isinstance(a, torch.Tensor):
            t = a.detach().to("cpu")
            if t.dtype == torch.bfloat16:
                t = t.to(torch.float32)
            a = t.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    return a.reshape((a.shape[0] * a.shape[1],) + a.shape[2:])


def _run_group(fn: Callable, args, kwargs):
    """Worker body: the oracle on one group of heads, laid out as B = 1."""
    call = [None if a is None else np.asarray(a, dtype=np.float64)[None] for a in args]
    out = fn(*call, **kwargs)
    return tuple(np.asarray(r)[0] for r in out)


def oracle_heads(fn: Callable, args: Sequence, heads: Optional[Sequence[tuple]] = None,
                 **kwargs):
    """``fn(*args, **kwargs)`` for an oracle function whose array arguments
    (``None`` allowed) all start with the (B, H) axes and whose results do too.

    ``heads``: the (b, h) pairs to run, or None for all of them.  Returns the
    results with a leading axis of 1 and the selected heads on axis 1 (for
    ``heads=None``: the full ``[B, H, ...]`` shape)."""
    flat = [_host(a) for a in args]
    B, H = next(tuple(a.shape[:2]) for a in args if a is not None)
    sel = list(range(B * H)) if heads is None else [b * H + h for b, h in heads]
    nw = n_workers(len(sel))
    groups = [g for g in np.array_split(np.asarray(sel), nw) if len(g)]
    jobs = [tuple(None if a is None else a[g] for a in flat) for g in groups]
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=len(jobs), mp_context=ctx) as ex:
        parts = list(ex.map(_run_group, [fn] * len(jobs), jobs, [kwargs] * len(jobs)))
    n_out = len(parts[0])
    outs = []
    for i in range(n_out):
        cat = np.concatenate([p[i] for p in parts], axis=0)
        if heads is None:
            cat = cat.reshape((B, H) + cat.shape[1:])
        else:
            cat = cat[None]
        outs.append(cat)
    return tuple(outs)


def features_forward(q_raw, k_raw, v, beta_logit, S0=None, alpha=None, dtype="bf16"):
    """The oracle's feature maps, then the plain (alpha None) or gated oracle
    forward on the mapped operands (a composition of oracle functions)."""
    from oracle import delta_rule_forward, feature_maps, gated_delta_rule_forward

    qh, kh, b = feature_maps(q_raw, k_raw, beta_logit, dtype)
    if alpha is None:
        return delta_rule_forward(qh, kh, v, b, S0)
    return gated_delta_rule_forward(qh, kh, v, alpha, b, S0)
