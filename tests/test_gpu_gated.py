"""Gated (Gated DeltaNet) chunked forward and decode step on the GPU, through
the C ABI, against the fp64 gated oracle."""

import sys

import numpy as np
import pytest
import torch

from deltanet_delta_rule_chunk_amd import inputs as I
from deltanet_delta_rule_chunk_amd.binding import chunk_fwd, gated_chunk_fwd, gated_decode_step
from oracle import gated_delta_rule_decode_step, gated_delta_rule_forward
from oracle_pool import oracle_heads
from parity import assert_parity, err_f32, record, to64, worst_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


def _run(x, alpha, C, out_dtype=torch.float32):
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    o, S = gated_chunk_fwd(g["q"], g["k"], g["v"], alpha.to(DEV), g["beta"], g["S0"], C,
                           out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def _oracle(x, alpha, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[[b for b, _ in heads], [h for _, h in heads]][None])
    q, k, v, beta = (sel(to64(x[n])) for n in ("q", "k", "v", "beta"))
    S0 = None if x["S0"] is None else sel(to64(x["S0"]))
    return gated_delta_rule_forward(q, k, v, sel(to64(alpha)), beta, S0)


SMALL = [
    # name, dtype, B, H, L, dk, dv, C, S0
    ("f32_d64_C64_L256", "f32", 1, 2, 256, 64, 64, 64, False),
    ("f32_d128_C128_ragged", "f32", 1, 2, 300, 128, 128, 128, True),
    ("f32_dk64_dv128_ragged", "f32", 2, 1, 200, 64, 128, 64, True),
    ("bf16_dk128_dv64_C128_ragged", "bf16", 1, 3, 333, 128, 64, 128, True),
    ("bf16_d64_C64_ragged", "bf16", 2, 2, 64 * 5 + 7, 64, 64, 64, False),
    ("bf16_d128_C64_S0", "bf16", 1, 2, 640, 128, 128, 64, True),
    ("bf16_d128_C128", "bf16", 1, 2, 512, 128, 128, 128, True),
    ("bf16_dk64_dv128_C128", "bf16", 1, 2, 384, 64, 128, 128, True),
    ("bf16_L_below_C", "bf16", 1, 2, 37, 128, 128, 128, True),
    ("bf16_L1_C128", "bf16", 1, 2, 1, 128, 128, 128, True),
    ("bf16_L129_C128", "bf16", 2, 1, 129, 128, 128, 128, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_gated_small_parity(gpu_lib, case):
    name, dt, B, H, L, dk, dv, C, s0 = case
    _note(f"[gated] {name}")
    w = I.ChunkWorkload(name, B, H, L, dk, dv, C, dt, s0_std=0.1 if s0 else None)
    x = I.make_chunk_inputs(w, seed=21)
    alpha = I.make_chunk_alpha(w, seed=21)
    o, S = _run(x, alpha, C)
    o_ref, S_ref = _oracle(x, alpha)
    assert_parity(o, o_ref, dt, f"{name} o")
    assert_parity(S, S_ref, dt, f"{name} S_final")


@pytest.mark.parametrize("dt,C", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_gated_alpha_one_equals_plain(gpu_lib, dt, C):
    """alpha = 1 is the plain delta rule: every decay factor is exactly 1.
    On the matrix-core (bf16) path the gated kernels then reproduce the plain
    kernels' bits.  The fp32 vector-ALU scan is compiled to a different
    multiply-add grouping once the decay multiplies are present (the plain
    one folds its sums into one fused chain), so there the two agree to
    rounding: measured 2e-7 of max|o|, checked at 2e-6."""
    w = I.ChunkWorkload("a1", 1, 2, 3 * C + 5, 128, 128, C, dt, s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=3)
    g = {k: t.to(DEV) for k, t in x.items()}
    ones = torch.ones_like(g["beta"])
    o1, S1 = gated_chunk_fwd(g["q"], g["k"], g["v"], ones, g["beta"], g["S0"], C)
    o2, S2 = chunk_fwd(g["q"], g["k"], g["v"], g["beta"], g["S0"], C)
    torch.cuda.synchronize()
    if dt == "bf16":
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
    else:
        assert float((o1 - o2).abs().max()) <= 2e-6 * float(o2.abs().max())
        assert float((S1 - S2).abs().max()) <= 2e-6 * float(S2.abs().max())


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gated_wipes_and_mixed_decays(gpu_lib, dt):
    """Exact zeros (full wipes), exact ones and small decays mixed within
    chunks, against the oracle (which applies alpha = 0 exactly)."""
    w = I.ChunkWorkload("wipe", 1, 2, 330, 128, 128, 128 if dt == "bf16" else 64, dt, s0_std=0.1)
    x = I.make_chunk_inputs(w, seed=4)
    alpha = I.make_chunk_alpha(w, seed=4)
    alpha[:, :, ::17] = 0.0
    alpha[:, :, 5::11] = 1.0
    alpha[:, 1, 40:60] = 0.05
    o, S = _run(x, alpha, w.C)
    o_ref, S_ref = _oracle(x, alpha)
    assert_parity(o, o_ref, dt, "o")
    assert_parity(S, S_ref, dt, "S_final")


def test_gated_long_context(gpu_lib):
    """The long-context shape (B=1, H=32, L=65536, d=128, C=128) with the gate,
    at full size on the GPU; every head against the gated oracle."""
    w = I.WORKLOADS[3]
    _note(f"[gated] {w.name}")
    x = I.make_chunk_inputs(w, seed=0)
    alpha = I.make_chunk_alpha(w, seed=0)
    o, S = _run(x, alpha, w.C)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    _note(f"  oracle on all {w.B * w.H} heads")
    o_ref, S_ref = oracle_heads(gated_delta_rule_forward,
                                (x["q"], x["k"], x["v"], alpha, x["beta"], x["S0"]))
    e = assert_parity(o, o_ref, "bf16", "o")
    eS = assert_parity(S, S_ref, "bf16", "S_final")
    wh = worst_head(o, o_ref)
    _note(f"  o err/RMS = {e:.3e} (worst head {wh}), S_final {eS:.3e}")
    record("gated_workload3", workload=w.name + "_gated", heads=w.B * w.H, o_f32_out=e,
           S_final=eS, worst_head_f32_out=wh)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gated_decode_small(gpu_lib, dt, dk, dv):
    w = I.DecodeWorkload("gd", 3, 5, dk, dv, 4, dt, 0.1)
    S = I.make_decode_state(w, seed=2)
    S_ref = to64(S)
    Sg = S.to(DEV)
    for step in range(w.steps):
        x = I.make_decode_step_inputs(w, step, seed=2)
        a = I.make_decode_alpha(w, step, seed=2)
        if step == 2:
            a[0] = 0.0
        o = gated_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), a.to(DEV),
                              x["beta"].to(DEV), Sg)
        torch.cuda.synchronize()
        o_ref, S_ref = gated_delta_rule_decode_step(to64(x["q"]), to64(x["k"]), to64(x["v"]),
                                                    to64(a), to64(x["beta"]), S_ref)
        assert_parity(o.cpu(), o_ref, dt, f"o step {step}")
    assert_parity(Sg.cpu(), S_ref, dt, "S")


def test_gated_decode_workload_first_steps(gpu_lib):
    """The decode workload's shape (B=256, H=32, d=128, 512 MiB of state) with
    the gate, on the full state for the first steps."""
    w = I.WORKLOADS[4]
    _note(f"[gated] {w.name}")
    S = I.make_decode_state(w, seed=0)
    S_ref = to64(S)
    Sg = S.to(DEV)
    for step in range(2):
        x = I.make_decode_step_inputs(w, step, seed=0)
        a = I.make_decode_alpha(w, step, seed=0)
        o = gated_decode_step(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), a.to(DEV),
                              x["beta"].to(DEV), Sg)
        torch.cuda.synchronize()
        o_ref, S_ref = gated_delta_rule_decode_step(to64(x["q"]), to64(x["k"]), to64(x["v"]),
                                                    to64(a), to64(x["beta"]), S_ref)
        assert_parity(o.cpu(), o_ref, "bf16", f"o step {step}")
    assert_parity(Sg.cpu(), S_ref, "bf16", "S")


# ---- properties of the gated path that hold at any size -------------------------

def _dev(x):
    return {k: (None if t is None else t.to(DEV)) for k, t in x.items()}


def test_gated_chunk_size_invariance(gpu_lib):
    """C = 64 and C = 128 compute the same gated recurrence (bf16 inputs)."""
    w = I.ChunkWorkload("gcinv", 1, 2, 1000, 128, 128, 64, "bf16", s0_std=0.1)
    g = _dev(I.make_chunk_inputs(w, seed=31))
    a = I.make_chunk_alpha(w, seed=31).to(DEV)
    o64, S64 = gated_chunk_fwd(g["q"], g["k"], g["v"], a, g["beta"], g["S0"], 64)
    o128, S128 = gated_chunk_fwd(g["q"], g["k"], g["v"], a, g["beta"], g["S0"], 128)
    torch.cuda.synchronize()
    assert_parity(o64.cpu(), o128.cpu(), "bf16", "o C64 vs C128")
    assert_parity(S64.cpu(), S128.cpu(), "bf16", "S C64 vs C128")


def test_gated_split_invariance(gpu_lib):
    """Two gated calls chained through S_final -> S0 equal one call (fp32), cut
    at a chunk boundary and off it: the decay restarts at every chunk start."""
    w = I.ChunkWorkload("gsplit", 2, 2, 384, 64, 64, 64, "f32", s0_std=0.1)
    g = _dev(I.make_chunk_inputs(w, seed=32))
    al = I.make_chunk_alpha(w, seed=32).to(DEV)
    o, S = gated_chunk_fwd(g["q"], g["k"], g["v"], al, g["beta"], g["S0"], 64)
    for cut in (128, 150):
        a = {k: g[k][:, :, :cut].contiguous() for k in ("q", "k", "v", "beta")}
        b = {k: g[k][:, :, cut:].contiguous() for k in ("q", "k", "v", "beta")}
        o1, S1 = gated_chunk_fwd(a["q"], a["k"], a["v"], al[:, :, :cut].contiguous(), a["beta"],
                                 g["S0"], 64)
        o2, S2 = gated_chunk_fwd(b["q"], b["k"], b["v"], al[:, :, cut:].contiguous(), b["beta"], S1, 64)
        torch.cuda.synchronize()
        assert err_f32(torch.cat([o1, o2], 2).cpu(), o.cpu()) < 1e-5
        assert err_f32(S2.cpu(), S.cpu()) < 1e-5


def test_gated_decode_equals_chunk(gpu_lib):
    """L gated decode steps equal one gated chunked forward over the same L tokens."""
    w = I.ChunkWorkload("gdvc", 2, 3, 70, 128, 64, 64, "f32", s0_std=0.1)
    g = _dev(I.make_chunk_inputs(w, seed=33))
    al = I.make_chunk_alpha(w, seed=33).to(DEV)
    o, S = gated_chunk_fwd(g["q"], g["k"], g["v"], al, g["beta"], g["S0"], 64)
    Sd = g["S0"].clone()
    outs = []
    for t in range(w.L):
        outs.append(gated_decode_step(*(g[n][:, :, t].contiguous() for n in ("q", "k", "v")),
                                      al[:, :, t].contiguous(), g["beta"][:, :, t].contiguous(), Sd))
    torch.cuda.synchronize()
    assert err_f32(torch.stack(outs, 2).cpu(), o.cpu()) < 1e-4
    assert err_f32(Sd.cpu(), S.cpu()) < 1e-4


def test_gated_linearity_in_values_and_state(gpu_lib):
    """For fixed q, k, alpha, beta the gated map (V, S0) -> (O, S_final) is linear."""
    w = I.ChunkWorkload("glin", 1, 2, 200, 64, 64, 64, "f32", s0_std=0.1)
    g1 = _dev(I.make_chunk_inputs(w, seed=34))
    g2 = _dev(I.make_chunk_inputs(w, seed=35))
    al = I.make_chunk_alpha(w, seed=34).to(DEV)
    a, b = 0.75, -1.5
    v = (a * g1["v"] + b * g2["v"]).contiguous()
    S0 = (a * g1["S0"] + b * g2["S0"]).contiguous()
    o, S = gated_chunk_fwd(g1["q"], g1["k"], v, al, g1["beta"], S0, 64)
    o1, S1 = gated_chunk_fwd(g1["q"], g1["k"], g1["v"], al, g1["beta"], g1["S0"], 64)
    o2, S2 = gated_chunk_fwd(g1["q"], g1["k"], g2["v"], al, g1["beta"], g2["S0"], 64)
    torch.cuda.synchronize()
    assert err_f32((a * o1 + b * o2).cpu(), o.cpu()) < 1e-4
    assert err_f32((a * S1 + b * S2).cpu(), S.cpu()) < 1e-4


def test_gated_bitwise_determinism(gpu_lib):
    w = I.ChunkWorkload("gdet", 2, 4, 1024, 128, 128, 128, "bf16", s0_std=0.1)
    g = _dev(I.make_chunk_inputs(w, seed=36))
    al = I.make_chunk_alpha(w, seed=36).to(DEV)
    o1, S1 = gated_chunk_fwd(g["q"], g["k"], g["v"], al, g["beta"], g["S0"], 128)
    o2, S2 = gated_chunk_fwd(g["q"], g["k"], g["v"], al, g["beta"], g["S0"], 128)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_gated_decay_only_on_gpu(gpu_lib):
    """beta = 0: only the decay acts, S_L = (alpha_1 ... alpha_L) S0 and
    o_t = (alpha_1 ... alpha_t) q_t S0 (bf16 path, long enough for 3 chunks)."""
    w = I.ChunkWorkload("gdecay", 1, 2, 300, 128, 128, 128, "bf16", s0_std=0.1)
    g = _dev(I.make_chunk_inputs(w, seed=37))
    al = I.make_chunk_alpha(w, seed=37)
    al = 0.5 + 0.5 * al                      # keep the products away from underflow
    beta = torch.zeros_like(g["beta"])
    o, S = gated_chunk_fwd(g["q"], g["k"], g["v"], al.to(DEV), beta, g["S0"], 128)
    torch.cuda.synchronize()
    cp = np.cumprod(to64(al), axis=-1)
    want_o = cp[..., None] * (to64(g["q"]) @ to64(g["S0"]))
    want_S = cp[:, :, -1, None, None] * to64(g["S0"])
    assert_parity(o.cpu(), want_o, "bf16", "o")
    assert_parity(S.cpu(), want_S, "bf16", "S")
