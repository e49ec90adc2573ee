"""Decode step on the GPU (through the C ABI) against the fp64 oracle."""

import sys

import numpy as np
import pytest
import torch

from deltanet_delta_rule_chunk_amd import inputs as I
from deltanet_delta_rule_chunk_amd.binding import decode_step, gated_decode_step, kda_decode_step
from oracle import delta_rule_decode_step, gated_delta_rule_decode_step, kda_delta_rule_decode_step
from parity import assert_parity, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_small(gpu_lib, dt, dk, dv):
    _note(f"[decode] small {dt} {dk}x{dv}")
    w = I.DecodeWorkload("small", 3, 5, dk, dv, 20, dt, 0.1)
    S = I.make_decode_state(w, seed=2)
    S_ref = to64(S)
    Sg = S.to(DEV)
    for step in range(w.steps):
        x = I.make_decode_step_inputs(w, step, seed=2)
        o = decode_step(*(x[n].to(DEV) for n in ("q", "k", "v", "beta")), Sg)
        o_ref, S_ref = delta_rule_decode_step(*(to64(x[n]) for n in ("q", "k", "v", "beta")), S_ref)
        torch.cuda.synchronize()
        assert_parity(o.cpu(), o_ref, dt, f"o step {step}")
    assert_parity(Sg.cpu(), S_ref, dt, "S")


def test_decode_bf16_output(gpu_lib):
    w = I.DecodeWorkload("small", 4, 4, 128, 128, 1, "bf16", 0.1)
    S = I.make_decode_state(w, seed=4)
    x = I.make_decode_step_inputs(w, 0, seed=4)
    o = decode_step(*(x[n].to(DEV) for n in ("q", "k", "v", "beta")), S.to(DEV),
                    out_dtype=torch.bfloat16)
    o_ref, _ = delta_rule_decode_step(*(to64(x[n]) for n in ("q", "k", "v", "beta")), to64(S))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    assert_parity(o.cpu(), o_ref, "bf16", "o")


def test_decode_workload_full_state_first_steps(gpu_lib):
    """B=256, H=32, d=128: the whole state against the oracle for 8 steps."""
    w = I.WORKLOADS[4]
    _note(f"[decode] {w.name} full state, 8 steps")
    S = I.make_decode_state(w, seed=0)
    S_ref = to64(S)
    Sg = S.to(DEV)
    for step in range(8):
        x = I.make_decode_step_inputs(w, step, seed=0)
        o = decode_step(*(x[n].to(DEV) for n in ("q", "k", "v", "beta")), Sg)
        o_ref, S_ref = delta_rule_decode_step(*(to64(x[n]) for n in ("q", "k", "v", "beta")), S_ref)
        torch.cuda.synchronize()
        assert_parity(o.cpu(), o_ref, "bf16", f"o step {step}")
    assert_parity(Sg.cpu(), S_ref, "bf16", "S after 8 steps")


@pytest.mark.timeout(400)
def test_decode_workload_1000_steps_head_subset(gpu_lib):
    """All 1000 steps at full size on the GPU; the oracle follows 64 seeded
    (b, h) heads (heads are independent, so the subset check is exact for
    them).  o is checked every step, S at the end."""
    w = I.WORKLOADS[4]
    _note(f"[decode] {w.name} 1000 steps, 64-head subset")
    rng = np.random.default_rng(99)
    flat = rng.choice(w.B * w.H, 64, replace=False)
    bi, hi = flat // w.H, flat % w.H
    S = I.make_decode_state(w, seed=0)
    S_ref = to64(S)[bi, hi][None]
    Sg = S.to(DEV)
    del S
    worst = 0.0
    for step in range(w.steps):
        x = I.make_decode_step_inputs(w, step, seed=0)
        o = decode_step(*(x[n].to(DEV, non_blocking=True) for n in ("q", "k", "v", "beta")), Sg)
        sub = [to64(x[n])[bi, hi][None] for n in ("q", "k", "v", "beta")]
        o_ref, S_ref = delta_rule_decode_step(*sub, S_ref)
        o_sub = o[torch.as_tensor(bi, device=DEV), torch.as_tensor(hi, device=DEV)].cpu()[None]
        worst = max(worst, assert_parity(o_sub, o_ref, "bf16", f"o step {step}"))
        if step % 200 == 0:
            _note(f"  step {step} worst err/RMS {worst:.3e}")
    S_sub = Sg[torch.as_tensor(bi, device=DEV), torch.as_tensor(hi, device=DEV)].cpu()[None]
    assert_parity(S_sub, S_ref, "bf16", "S after 1000 steps")


@pytest.mark.parametrize("form", ["plain", "gated", "kda"])
def test_decode_ragged_heads_per_workgroup(gpu_lib, form):
    """B * H = 805 heads: the persistent workgroups (one per CU) walk three or
    four heads each, with the next two heads' state loads in flight, so the
    end of every walk is exercised; three successive steps against the
    oracle on every head."""
    _note(f"[decode] ragged heads, {form}")
    w = I.DecodeWorkload("ragged", 35, 23, 128, 128, 3, "bf16", 0.1)
    S = I.make_decode_state(w, seed=9)
    S_ref = to64(S)
    Sg = S.to(DEV)
    for step in range(w.steps):
        x = I.make_decode_step_inputs(w, step, seed=9)
        args = [x[n].to(DEV) for n in ("q", "k", "v")]
        ref_args = [to64(x[n]) for n in ("q", "k", "v")]
        if form == "plain":
            o = decode_step(*args, x["beta"].to(DEV), Sg)
            o_ref, S_ref = delta_rule_decode_step(*ref_args, to64(x["beta"]), S_ref)
        elif form == "gated":
            a = I.make_decode_alpha(w, step, seed=9)
            o = gated_decode_step(*args, a.to(DEV), x["beta"].to(DEV), Sg)
            o_ref, S_ref = gated_delta_rule_decode_step(*ref_args, to64(a), to64(x["beta"]), S_ref)
        else:
            a = I.make_decode_kda_alpha(w, step, seed=9)
            o = kda_decode_step(*args, a.to(DEV), x["beta"].to(DEV), Sg)
            o_ref, S_ref = kda_delta_rule_decode_step(*ref_args, to64(a), to64(x["beta"]), S_ref)
        torch.cuda.synchronize()
        assert_parity(o.cpu(), o_ref, "bf16", f"{form} o step {step}")
    assert_parity(Sg.cpu(), S_ref, "bf16", f"{form} S")

