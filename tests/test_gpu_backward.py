"""Gradient of the chunked forward on the GPU (deltanet_chunk_bwd), through
the C ABI, against the fp64 backward oracle (oracle/backward.py), and, at
the full long-context size where the oracle would need every state, against
identities that hold exactly at any size."""

import sys

import numpy as np
import pytest
import torch

from deltanet_delta_rule_chunk_amd import inputs as I
from deltanet_delta_rule_chunk_amd.binding import chunk_bwd, chunk_fwd, delta_rule
from oracle import delta_rule_backward
from oracle_pool import oracle_heads
from parity import assert_parity, record, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dbeta", "dS0")


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


def _grads_in(w, seed, dsf=True):
    """Seeded output gradients: dO ~ N(0, 1), dS_final ~ N(0, 0.01)."""
    rng = np.random.default_rng([seed, 17])
    dO = torch.from_numpy(rng.standard_normal((w.B, w.H, w.L, w.d_v))).to(torch.float32)
    dSf = (torch.from_numpy(rng.standard_normal((w.B, w.H, w.d_k, w.d_v)) * 0.1).to(torch.float32)
           if dsf else None)
    return dO, dSf


def _oracle(x, dO, dSf, heads=None):
    sel = (lambda t: t) if heads is None else (
        lambda t: t[[b for b, _ in heads], [h for _, h in heads]][None])
    q, k, v, beta = (sel(to64(x[n])) for n in ("q", "k", "v", "beta"))
    S0 = None if x["S0"] is None else sel(to64(x["S0"]))
    return delta_rule_backward(q, k, v, beta, S0, sel(to64(dO)),
                               None if dSf is None else sel(to64(dSf)))


def _run(x, dO, dSf, C):
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    out = chunk_bwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], dO.to(DEV),
                    None if dSf is None else dSf.to(DEV), C)
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


SMALL = [
    # name, dtype, B, H, L, dk, dv, C, S0, dS_final
    ("f32_d64_L256", "f32", 1, 2, 256, 64, 64, 64, False, False),
    ("f32_d128_ragged_states", "f32", 1, 2, 300, 128, 128, 128, True, True),
    ("f32_dk64_dv128_ragged", "f32", 2, 1, 200, 64, 128, 64, True, False),
    ("f32_dk128_dv64", "f32", 1, 2, 192, 128, 64, 64, False, True),
    ("bf16_d64_ragged", "bf16", 2, 2, 64 * 5 + 7, 64, 64, 64, True, True),
    ("bf16_d128_states", "bf16", 1, 2, 640, 128, 128, 128, True, True),
    ("bf16_L_below_chunk", "bf16", 1, 2, 37, 128, 128, 64, True, True),
    ("bf16_dk64_dv128_ragged", "bf16", 3, 3, 64 * 3 + 19, 64, 128, 64, True, True),
    ("bf16_dk128_dv64_nine_heads", "bf16", 1, 9, 64 * 4, 128, 64, 128, False, True),
    # an odd number of 64-token blocks: the forward pass's last 128-token
    # chunk has no second block
    ("bf16_d128_odd_blocks", "bf16", 1, 2, 64 * 4 + 21, 128, 128, 64, True, True),
    # one token; exactly one 64-token block; a second block of one row; a
    # last 128-token chunk of one row
    ("bf16_d128_one_token", "bf16", 1, 2, 1, 128, 128, 64, True, True),
    ("bf16_d64_one_block", "bf16", 1, 3, 64, 64, 64, 64, False, True),
    ("bf16_d128_L65", "bf16", 1, 2, 65, 128, 128, 128, True, False),
    ("bf16_d128_L129", "bf16", 2, 1, 129, 128, 128, 64, True, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_backward_small_parity(gpu_lib, case):
    name, dt, B, H, L, dk, dv, C, s0, dsf = case
    _note(f"[bwd] {name}")
    w = I.ChunkWorkload(name, B, H, L, dk, dv, C, dt, s0_std=0.1 if s0 else None)
    x = I.make_chunk_inputs(w, seed=41)
    dO, dSf = _grads_in(w, 41, dsf)
    got = _run(x, dO, dSf, C)
    ref = _oracle(x, dO, dSf)
    for n, a, b in zip(NAMES, got, ref):
        e = assert_parity(a, b, dt, f"{name} {n}")
        _note(f"  {n} err = {e:.2e}")


def test_backward_gpt2_heads_sampled(gpu_lib):
    """B = 4, H = 12, L = 2048, d = 64 at full size; the oracle on three
    sampled heads."""
    w = I.WORKLOADS[1]
    x = I.make_chunk_inputs(w, seed=0)
    dO, dSf = _grads_in(w, 0)
    got = _run(x, dO, dSf, w.C)
    heads = [(0, 0), (2, 7), (3, 11)]
    ref = _oracle(x, dO, dSf, heads)
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    for n, a, b in zip(NAMES, got, ref):
        assert_parity(a[bi, hi][None], b, "bf16", n)


def test_backward_overwrite_heads_sampled(gpu_lib):
    """B = 2, H = 16, L = 8192, d = 128, S0 given, beta = 1 on heads 0-7; the
    oracle on one head from each half."""
    w = I.WORKLOADS[2]
    x = I.make_chunk_inputs(w, seed=0)
    dO, dSf = _grads_in(w, 0)
    got = _run(x, dO, dSf, w.C)
    heads = [(0, 3), (1, 12)]
    ref = _oracle(x, dO, dSf, heads)
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    for n, a, b in zip(NAMES, got, ref):
        assert_parity(a[bi, hi][None], b, "bf16", n)


def test_backward_empty_sequence(gpu_lib):
    w = I.ChunkWorkload("empty", 1, 2, 0, 64, 64, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=1)
    dO, dSf = _grads_in(w, 1)
    dq, dk, dv, db, dS0 = _run(x, dO, dSf, 64)
    assert dq.numel() == 0 and torch.equal(dS0, dSf)


def test_backward_long_context_identities(gpu_lib):
    """L = 65536, 32 heads of d = 128 at full size.  o and S_final are linear
    in q, and jointly linear in (v, S0), so (Euler) for any dO, dS_final:
        <dq, q> = <dO, o>,   <dv, v> + <dS0, S0> = <dO, o> + <dS_final, S_final>,
    with o, S_final from the forward kernels (checked to 1e-4 of the sum of
    the terms' magnitudes)."""
    w = I.scaled_chunk_workload(I.WORKLOADS[3], s0_std=0.1)
    _note(f"[bwd] {w.name} with S0")
    x = I.make_chunk_inputs(w, seed=0)
    dO, dSf = _grads_in(w, 0)
    g = {k: t.to(DEV) for k, t in x.items()}
    o, S = chunk_fwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], w.C)
    dq, dk, dv, db, dS0 = chunk_bwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], dO.to(DEV),
                                    dSf.to(DEV), w.C)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, db, dS0):
        assert torch.isfinite(t).all()
    dOd, dSfd = dO.to(DEV, torch.float64), dSf.to(DEV, torch.float64)
    lo = torch.sum(dOd * o.double()).item()
    ls = torch.sum(dSfd * S.double()).item()
    q_side = torch.sum(dq.double() * g["q"].double()).item()
    v_side = (torch.sum(dv.double() * g["v"].double()) + torch.sum(dS0.double() * g["S0"].double())).item()
    scale_q = torch.sum(torch.abs(dq.double() * g["q"].double())).item()
    scale_v = (torch.sum(torch.abs(dv.double() * g["v"].double())) +
               torch.sum(torch.abs(dS0.double() * g["S0"].double()))).item()
    _note(f"  <dq,q> {q_side:.6e} vs <dO,o> {lo:.6e}; <dv,v>+<dS0,S0> {v_side:.6e} vs {lo + ls:.6e}")
    assert abs(q_side - lo) <= 1e-4 * scale_q
    assert abs(v_side - (lo + ls)) <= 1e-4 * scale_v


def test_backward_long_context_elementwise(gpu_lib):
    """L = 65536, 32 heads of d = 128 at full size on the GPU, every gradient
    element-wise against the fp64 backward oracle on four heads spread over
    the head range (the oracle keeps all L + 1 states of a head in fp64,
    8.6 GB each, so it runs one head per worker process)."""
    w = I.WORKLOADS[3]
    _note(f"[bwd] {w.name} element-wise, four heads")
    x = I.make_chunk_inputs(w, seed=0)
    dO, dSf = _grads_in(w, 0)
    got = _run(x, dO, dSf, w.C)
    heads = [(0, 0), (0, 9), (0, 21), (0, 31)]
    ref = oracle_heads(delta_rule_backward, (x["q"], x["k"], x["v"], x["beta"], x["S0"], dO, dSf),
                       heads)
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    errs = {}
    for n, a, b in zip(NAMES, got, ref):
        errs[n] = assert_parity(a[bi, hi][None], b, "bf16", n)
    _note("  " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    record("backward_workload3", workload=w.name + "_backward", heads=heads, **errs)


def test_backward_bitwise_determinism(gpu_lib):
    """Two runs of the same gradient give identical bits (no atomics or
    order-dependent reductions anywhere in the backward)."""
    w = I.ChunkWorkload("det", 2, 5, 64 * 6 + 21, 128, 128, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=8)
    dO, dSf = _grads_in(w, 8)
    a = _run(x, dO, dSf, 64)
    b = _run(x, dO, dSf, 64)
    for n, ga, gb in zip(NAMES, a, b):
        assert torch.equal(ga, gb), n



@pytest.mark.parametrize("dtype,with_s0", [("f32", True), ("bf16", True), ("bf16", False)])
def test_autograd_matches_chunk_bwd(gpu_lib, dtype, with_s0):
    """delta_rule under autograd: its outputs are chunk_fwd's and the
    gradients it hands back are chunk_bwd's for the same output gradients
    (cast by autograd to each input's dtype), bit for bit."""
    _note(f"[bwd] autograd {dtype} S0={with_s0}")
    w = I.ChunkWorkload("ag", 1, 3, 64 * 3 + 29, 64, 64, 64, dtype, s0_std=0.1 if with_s0 else None)
    x = I.make_chunk_inputs(w, seed=12)
    dO, dSf = _grads_in(w, 12)
    g = {n: (None if t is None else t.to(DEV)) for n, t in x.items()}
    leaves = {n: (None if t is None else t.clone().requires_grad_(True)) for n, t in g.items()}
    o, S_final = delta_rule(leaves["q"], leaves["k"], leaves["v"], leaves["beta"], leaves["S0"], 64)
    o_ref, S_ref = chunk_fwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], 64)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref) and torch.equal(S_final.detach(), S_ref)
    ((o * dO.to(DEV)).sum() + (S_final * dSf.to(DEV)).sum()).backward()
    ref = chunk_bwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], dO.to(DEV), dSf.to(DEV), 64)
    torch.cuda.synchronize()
    for n, r in zip(("q", "k", "v", "beta", "S0"), ref):
        if leaves[n] is None:
            continue
        got = leaves[n].grad
        assert got is not None and got.dtype == leaves[n].dtype, n
        assert torch.equal(got, r.to(got.dtype)), n
