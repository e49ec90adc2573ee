"""Per-dimension decay (KDA) chunked forward and decode step on the GPU,
through the C ABI, against the fp64 KDA oracle (oracle/kda.py)."""

import sys

import numpy as np
import pytest
import torch

from deltanet_delta_rule_chunk_amd import inputs as I
from deltanet_delta_rule_chunk_amd.binding import (chunk_fwd, gated_chunk_fwd, kda_chunk_fwd,
                                                   kda_decode_step)
from oracle import kda_delta_rule_decode_step, kda_delta_rule_forward
from oracle_pool import oracle_heads
from parity import assert_parity, record, to64, worst_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


def _oracle(x, alpha, heads=None, L=None):
    sel = (lambda t: t) if heads is None else (
        lambda t: t[[b for b, _ in heads], [h for _, h in heads]][None])
    cut = (lambda t: t) if L is None else (lambda t: t[:, :, :L])
    q, k, v, beta = (cut(sel(to64(x[n]))) for n in ("q", "k", "v", "beta"))
    S0 = None if x["S0"] is None else sel(to64(x["S0"]))
    return kda_delta_rule_forward(q, k, v, cut(sel(to64(alpha))), beta, S0)


SMALL = [
    # name, dtype, B, H, L, dk, dv, C, S0
    ("f32_d64_L256", "f32", 1, 2, 256, 64, 64, 64, False),
    ("f32_d128_ragged_S0", "f32", 1, 2, 300, 128, 128, 128, True),
    ("f32_dk64_dv128_ragged", "f32", 2, 1, 200, 64, 128, 64, True),
    ("bf16_dk128_dv64_ragged_S0", "bf16", 1, 3, 333, 128, 64, 128, True),
    ("bf16_d64_ragged", "bf16", 2, 2, 64 * 5 + 7, 64, 64, 64, False),
    ("bf16_d128_S0", "bf16", 1, 2, 640, 128, 128, 64, True),
    ("bf16_L_below_chunk", "bf16", 1, 2, 37, 128, 128, 128, True),
    ("bf16_L1", "bf16", 1, 2, 1, 128, 128, 128, True),
    ("bf16_L65", "bf16", 2, 1, 65, 128, 128, 64, True),
    ("bf16_dk64_dv128_ragged", "bf16", 3, 3, 64 * 4 + 50, 64, 128, 64, True),
    ("bf16_d128_nine_heads", "bf16", 1, 9, 64 * 3, 128, 128, 128, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_kda_small_parity(gpu_lib, case):
    name, dt, B, H, L, dk, dv, C, s0 = case
    _note(f"[kda] {name}")
    w = I.ChunkWorkload(name, B, H, L, dk, dv, C, dt, s0_std=0.1 if s0 else None)
    x = I.make_chunk_inputs(w, seed=31)
    alpha = I.make_chunk_kda_alpha(w, seed=31)
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    o, S = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha.to(DEV), g["beta"], g["S0"], C)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(x, alpha)
    e = assert_parity(o.cpu(), o_ref, dt, f"{name} o")
    assert_parity(S.cpu(), S_ref, dt, f"{name} S_final")
    _note(f"  o err = {e:.3e}")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_kda_bf16_output_is_rounded_fp32_output(gpu_lib, dk, dv):
    """The bf16 output of the same forward is the fp32 output rounded to
    nearest even (only the final store differs), and it meets the bf16 bar."""
    w = I.ChunkWorkload("kda_bf16_out", 2, 3, 64 * 3 + 5, dk, dv, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=12)
    alpha = I.make_chunk_kda_alpha(w, seed=12)
    g = {k: t.to(DEV) for k, t in x.items()}
    o32, S32 = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha.to(DEV), g["beta"], g["S0"], 64)
    o16, S16 = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha.to(DEV), g["beta"], g["S0"], 64,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16.cpu(), o32.cpu().to(torch.bfloat16))
    assert torch.equal(S16.cpu(), S32.cpu())
    o_ref, _ = _oracle(x, alpha)
    assert_parity(o16.cpu().float(), o_ref, "bf16", "kda bf16 o")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_kda_reductions_on_gpu(gpu_lib, dt):
    """All-ones gates give the plain forward; a gate equal in every dimension
    gives the scalar gated forward (different kernels: to the parity bar)."""
    w = I.ChunkWorkload("red", 1, 2, 2 * 128 + 19, 128, 128, 128, dt, s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=4)
    g = {k: t.to(DEV) for k, t in x.items()}
    ones = torch.ones(1, 2, w.L, 128, device=DEV)
    o1, S1 = kda_chunk_fwd(g["q"], g["k"], g["v"], ones, g["beta"], g["S0"], 128)
    o2, S2 = chunk_fwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], 128)
    a = I.make_chunk_alpha(w, seed=4).to(DEV)
    o3, S3 = kda_chunk_fwd(g["q"], g["k"], g["v"], a[..., None].expand(-1, -1, -1, 128).contiguous(),
                           g["beta"], g["S0"], 128)
    o4, S4 = gated_chunk_fwd(g["q"], g["k"], g["v"], a, g["beta"], g["S0"], 128)
    torch.cuda.synchronize()
    assert_parity(o1.cpu(), to64(o2.cpu()), dt, "ones vs plain o")
    assert_parity(S1.cpu(), to64(S2.cpu()), dt, "ones vs plain S")
    assert_parity(o3.cpu(), to64(o4.cpu()), dt, "constant vector vs scalar gate o")
    assert_parity(S3.cpu(), to64(S4.cpu()), dt, "constant vector vs scalar gate S")


def test_kda_wipes_and_exact_zeros(gpu_lib):
    """Gates with exact zeros in some dimensions (a per-dimension wipe) and
    ones in others, on a ragged length."""
    w = I.ChunkWorkload("wipe", 1, 2, 150, 64, 64, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=8)
    alpha = I.make_chunk_kda_alpha(w, seed=8)
    alpha[:, :, ::7, :16] = 0.0
    alpha[:, :, 3::11, 16:32] = 1.0
    alpha[:, :, 100, :] = 0.0
    g = {k: t.to(DEV) for k, t in x.items()}
    o, S = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha.to(DEV), g["beta"], g["S0"], 64)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(x, alpha)
    assert_parity(o.cpu(), o_ref, "bf16", "o")
    assert_parity(S.cpu(), S_ref, "bf16", "S_final")


def test_kda_empty_sequence_copies_state(gpu_lib):
    w = I.ChunkWorkload("empty", 1, 2, 0, 64, 64, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=1)
    g = {k: t.to(DEV) for k, t in x.items()}
    o, S = kda_chunk_fwd(g["q"], g["k"], g["v"], torch.empty(1, 2, 0, 64, device=DEV), g["beta"],
                         g["S0"], 64)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, g["S0"])


def test_kda_long_context(gpu_lib):
    """L = 65536, 32 heads of d = 128 at full size; every head against the
    KDA oracle over the whole sequence."""
    w = I.WORKLOADS[3]
    _note(f"[kda] {w.name}")
    x = I.make_chunk_inputs(w, seed=0)
    alpha = I.make_chunk_kda_alpha(w, seed=0)
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    o, S = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha.to(DEV), g["beta"], None, w.C)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    o, S = o.cpu(), S.cpu()
    del g
    _note(f"  oracle on all {w.B * w.H} heads")
    o_ref, S_ref = oracle_heads(kda_delta_rule_forward,
                                (x["q"], x["k"], x["v"], alpha, x["beta"], None))
    e = assert_parity(o, o_ref, "bf16", "o")
    eS = assert_parity(S, S_ref, "bf16", "S_final")
    wh = worst_head(o, o_ref)
    _note(f"  o err/RMS = {e:.3e} (worst head {wh}), S_final {eS:.3e}")
    record("kda_workload3", workload=w.name + "_kda", heads=w.B * w.H, o_f32_out=e, S_final=eS,
           worst_head_f32_out=wh)


@pytest.mark.parametrize("dt,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("f32", 128, 64),
                                      ("f32", 64, 64)])
def test_kda_decode_parity(gpu_lib, dt, dk, dv):
    """Eight steps in a row with the state carried."""
    w = I.DecodeWorkload("kdec", 3, 5, dk, dv, 8, dt, 0.1)
    _note(f"[kda] decode {dt} {dk}x{dv}")
    S = I.make_decode_state(w, seed=6)
    S_dev = S.to(DEV)
    S_ref = to64(S)
    for step in range(w.steps):
        x = I.make_decode_step_inputs(w, step, seed=6)
        a = I.make_decode_kda_alpha(w, step, seed=6)
        if step == 3:
            a[:, :, ::5] = 0.0  # exact per-dimension wipes
        o = kda_decode_step(*(x[n].to(DEV) for n in ("q", "k", "v")), a.to(DEV),
                            x["beta"].to(DEV), S_dev)
        o_ref, S_ref = kda_delta_rule_decode_step(*(to64(x[n]) for n in ("q", "k", "v")), to64(a),
                                                  to64(x["beta"]), S_ref)
        torch.cuda.synchronize()
        assert_parity(o.cpu(), o_ref, dt, f"step {step} o")
    assert_parity(S_dev.cpu(), S_ref, dt, "S after 8 steps")


def test_kda_decode_workload_first_steps(gpu_lib):
    """The decode workload at full size (B = 256, H = 32, d = 128): the whole
    512 MiB state against the oracle over two steps."""
    w = I.WORKLOADS[4]
    S = I.make_decode_state(w, seed=0)
    S_dev = S.to(DEV)
    S_ref = to64(S)
    del S
    for step in range(2):
        x = I.make_decode_step_inputs(w, step, seed=0)
        a = I.make_decode_kda_alpha(w, step, seed=0)
        o = kda_decode_step(*(x[n].to(DEV) for n in ("q", "k", "v")), a.to(DEV),
                            x["beta"].to(DEV), S_dev)
        o_ref, S_ref = kda_delta_rule_decode_step(*(to64(x[n]) for n in ("q", "k", "v")), to64(a),
                                                  to64(x["beta"]), S_ref)
        torch.cuda.synchronize()
        assert_parity(o.cpu(), o_ref, "bf16", f"step {step} o")
    assert_parity(S_dev.cpu(), S_ref, "bf16", "S")


def test_kda_decode_matches_chunk(gpu_lib):
    """T decode steps from S0 and one chunked forward over the same T tokens
    reach the same outputs and state."""
    B, H, T, d = 2, 3, 70, 128
    w = I.ChunkWorkload("dvc", B, H, T, d, d, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=9)
    a = I.make_chunk_kda_alpha(w, seed=9).to(DEV)
    g = {k: t.to(DEV) for k, t in x.items()}
    o_c, S_c = kda_chunk_fwd(g["q"], g["k"], g["v"], a, g["beta"], g["S0"], 64)
    S = g["S0"].clone()
    outs = [kda_decode_step(g["q"][:, :, t].contiguous(), g["k"][:, :, t].contiguous(),
                            g["v"][:, :, t].contiguous(), a[:, :, t].contiguous(),
                            g["beta"][:, :, t].contiguous(), S) for t in range(T)]
    torch.cuda.synchronize()
    assert_parity(torch.stack(outs, dim=2).cpu(), to64(o_c.cpu()), "bf16", "decode vs chunk o")
    assert_parity(S.cpu(), to64(S_c.cpu()), "bf16", "decode vs chunk S")


def test_kda_bitwise_determinism(gpu_lib):
    """Two runs of the same per-dimension-decay forward give identical bits."""
    w = I.ChunkWorkload("kda_det", 2, 5, 64 * 5 + 9, 128, 128, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=6)
    alpha = I.make_chunk_kda_alpha(w, seed=6).to(DEV)
    g = {k: t.to(DEV) for k, t in x.items()}
    o1, S1 = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha, g["beta"], g["S0"], 64)
    o2, S2 = kda_chunk_fwd(g["q"], g["k"], g["v"], alpha, g["beta"], g["S0"], 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)

