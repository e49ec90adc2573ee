"""The layer's feature maps on the GPU (the streaming feature kernel, the
chunked forward fed by raw projections, the decode step that maps in-kernel),
through the C ABI, against the fp64 oracle (oracle/features.py, then the
delta-rule oracle on the mapped operands).

Element-wise bar of the maps themselves.  The kernel evaluates them in fp32
with the hardware exp2 and reciprocal: for inputs of |x| <= 8 each output is
within DELTA = 4e-6 (relative) of the exact value (a bound summed from the
steps: the rounded exponent |x| 2^-24, exp2 and reciprocal ~1 ulp each, the
row's fp32 sum of squares, sqrt and division).  fp32 outputs must lie within
that of the exact map.  bf16 outputs are the exact map rounded to nearest
even, except where the exact value lies within DELTA of a rounding midpoint;
there the neighbouring bf16 value is accepted too (what is unique is checked:
every other element must match the oracle's rounding bit for bit).
"""

import sys

import numpy as np
import pytest
import torch

from deltanet_delta_rule_chunk_amd import inputs as I
from deltanet_delta_rule_chunk_amd.binding import chunk_fwd, decode_step, feature_prep
from oracle import (delta_rule_decode_step, delta_rule_forward, feature_maps,
                    gated_delta_rule_decode_step, gated_delta_rule_forward, round_to_bf16)
from oracle_pool import features_forward, oracle_heads
from parity import assert_parity, check_bf16_out, record, to64, worst_head

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DELTA = 4e-6
TINY = 1e-20  # rows in the eps branch map to ~|x| / 1e-12: absolute floor


def _note(msg):
    print(msg, file=sys.stderr, flush=True)


def _bf16_ulp(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e, -126) - 7), 2.0 ** -133)


def _check_map(got, exact, dtype, what, max_frac=0.01):
    """``got``: kernel output; ``exact``: the oracle's fp64 map (unrounded).
    ``max_frac`` bounds the share of near-tie bf16 elements (random inputs
    only: an underflowing row differs from the oracle in every element)."""
    g = to64(got)
    if dtype == "f32":
        err = np.abs(g - exact)
        bad = err > DELTA * np.abs(exact) + TINY
        assert not bad.any(), f"{what}: {bad.sum()} elements off by > {DELTA} rel (max {err.max():.3e})"
        return
    want = round_to_bf16(exact)
    differ = g != want
    allowed = np.abs(g - exact) <= 0.5 * _bf16_ulp(exact) + DELTA * np.abs(exact) + TINY
    bad = differ & ~allowed
    assert not bad.any(), f"{what}: {bad.sum()} elements neither the oracle's rounding nor a near-tie"
    frac = differ.mean()
    assert max_frac is None or frac < max_frac, \
        f"{what}: {frac:.4f} of the elements differ from the oracle's rounding"


def _exact_maps(x):
    """The oracle's exact (unrounded) q_hat, k_hat, beta."""
    return feature_maps(to64(x["q_raw"]), to64(x["k_raw"]), to64(x["beta_logit"]), "f64")


@pytest.mark.parametrize("dt,dk", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_feature_prep_elementwise(gpu_lib, dt, dk):
    # B H L = 2 * 3 * 257 rows: not a multiple of any workgroup's row count.
    w = I.ChunkWorkload("feat", 2, 3, 257, dk, 64, 64, dt)
    _note(f"[features] prep {dt} d_k={dk}")
    x = I.make_chunk_raw_inputs(w, seed=5)
    qh, kh, b = feature_prep(x["q_raw"].to(DEV), x["k_raw"].to(DEV), x["beta_logit"].to(DEV))
    torch.cuda.synchronize()
    eq, ek, eb = _exact_maps(x)
    _check_map(qh.cpu(), eq, dt, "q_hat")
    _check_map(kh.cpu(), ek, dt, "k_hat")
    err_b = np.abs(to64(b.cpu()) - eb).max()
    assert err_b <= 2e-6, f"beta: max err {err_b:.3e}"
    assert qh.dtype == x["q_raw"].dtype and b.dtype == torch.float32


def test_feature_prep_edge_rows(gpu_lib):
    """Zero rows (eps branch: zeros out), rows whose silu underflows (x = -100:
    e^{100} overflows fp32, silu -> -0), large positive rows (silu(x) = x),
    a single nonzero, mixed signs."""
    rows = np.zeros((12, 128))
    rows[1] = -100.0
    rows[2] = 60.0
    rows[3, 5] = 2.5
    rows[4, ::2], rows[4, 1::2] = 3.0, -3.0
    rows[5] = np.linspace(-8, 8, 128)
    rows[6, :64] = -100.0
    rows[6, 64] = 1.0
    rows[7:] = np.random.default_rng(9).standard_normal((5, 128)) * 4
    for dt, tdt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        q = torch.from_numpy(rows).to(tdt).reshape(1, 1, 12, 128)
        logit = torch.tensor([[[0.0, -100.0, 100.0, 3.0, -3.0, 0.5, -0.5, 8, -8, 1, 2, 3]]],
                             dtype=torch.float32)
        qh, kh, b = feature_prep(q.to(DEV), q.flip(2).contiguous().to(DEV), logit.to(DEV))
        torch.cuda.synchronize()
        eq, ek, eb = feature_maps(to64(q), to64(q.flip(2)), to64(logit), "f64")
        _check_map(qh.cpu(), eq, dt, f"{dt} q_hat edge rows", max_frac=None)
        _check_map(kh.cpu(), ek, dt, f"{dt} k_hat edge rows", max_frac=None)
        assert torch.all(qh[0, 0, 0] == 0) and torch.all(qh[0, 0, 1] == 0)
        assert np.abs(to64(b.cpu()) - eb).max() <= 2e-6
        assert torch.isfinite(qh).all() and torch.isfinite(b).all()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_feature_prep_in_place(gpu_lib, dt):
    w = I.ChunkWorkload("feat", 1, 2, 300, 128, 64, 64, dt)
    x = I.make_chunk_raw_inputs(w, seed=8)
    g = [x[n].to(DEV) for n in ("q_raw", "k_raw", "beta_logit")]
    ref = feature_prep(*g)
    got = feature_prep(*[t.clone() for t in g], in_place=True)
    torch.cuda.synchronize()
    for a, r in zip(got, ref):
        assert torch.equal(a, r)


FWD = [
    # name, dtype, B, H, L, dk, dv, C, S0, gated
    ("f32_d64_C64", "f32", 1, 2, 256, 64, 64, 64, False, False),
    ("f32_d128_C128_ragged_S0_gated", "f32", 1, 2, 300, 128, 128, 128, True, True),
    ("bf16_d64_C64_ragged", "bf16", 2, 2, 64 * 5 + 7, 64, 64, 64, False, False),
    ("bf16_d128_C128_S0", "bf16", 1, 2, 512, 128, 128, 128, True, False),
    ("bf16_dk128_dv64_C64_gated", "bf16", 1, 3, 333, 128, 64, 64, True, True),
    ("bf16_d128_C128_gated", "bf16", 1, 2, 640, 128, 128, 128, False, True),
]


def _fwd_oracle(x, dt, alpha=None, heads=None):
    sel = (lambda a: a) if heads is None else (
        lambda a: a[[b for b, _ in heads], [h for _, h in heads]][None])
    q, k, bl = (sel(to64(x[n])) for n in ("q_raw", "k_raw", "beta_logit"))
    qh, kh, b = feature_maps(q, k, bl, dt)
    v = sel(to64(x["v"]))
    S0 = None if x["S0"] is None else sel(to64(x["S0"]))
    if alpha is None:
        return delta_rule_forward(qh, kh, v, b, S0)
    return gated_delta_rule_forward(qh, kh, v, sel(to64(alpha)), b, S0)


@pytest.mark.parametrize("case", FWD, ids=lambda c: c[0])
def test_chunk_fwd_features_parity(gpu_lib, case):
    name, dt, B, H, L, dk, dv, C, s0, gated = case
    _note(f"[features] chunk {name}")
    w = I.ChunkWorkload(name, B, H, L, dk, dv, C, dt, s0_std=0.1 if s0 else None)
    x = I.make_chunk_raw_inputs(w, seed=13)
    alpha = I.make_chunk_alpha(w, seed=13) if gated else None
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    o, S = chunk_fwd(g["q_raw"], g["k_raw"], g["v"], g["beta_logit"], g["S0"], C,
                     alpha=None if alpha is None else alpha.to(DEV), features=True)
    torch.cuda.synchronize()
    o_ref, S_ref = _fwd_oracle(x, dt, alpha)
    e = assert_parity(o.cpu(), o_ref, dt, f"{name} o")
    assert_parity(S.cpu(), S_ref, dt, f"{name} S_final")
    _note(f"  o err = {e:.3e}")


@pytest.mark.parametrize("dt,gated,dk,dv,C,L", [
    ("bf16", False, 128, 128, 128, 2 * 128 + 9), ("bf16", True, 128, 128, 128, 2 * 128 + 9),
    ("bf16", False, 64, 64, 64, 3 * 64 + 1), ("bf16", True, 64, 128, 128, 100),
    ("bf16", False, 128, 64, 64, 5 * 64), ("f32", False, 128, 128, 128, 2 * 128 + 9)])
def test_chunk_fwd_features_is_maps_then_core(gpu_lib, dt, gated, dk, dv, C, L):
    """The fused call gives bit for bit what the feature prep followed by the
    core on its outputs gives: the bf16 path applies the maps inside its
    WY-prep kernel with the streaming kernel's arithmetic, the fp32 path runs
    the streaming kernel itself."""
    w = I.ChunkWorkload("two", 1, 2, L, dk, dv, C, dt, s0_std=0.1)
    x = I.make_chunk_raw_inputs(w, seed=2)
    g = {k: t.to(DEV) for k, t in x.items()}
    alpha = I.make_chunk_alpha(w, seed=2).to(DEV) if gated else None
    o1, S1 = chunk_fwd(g["q_raw"], g["k_raw"], g["v"], g["beta_logit"], g["S0"], C,
                       alpha=alpha, features=True)
    qh, kh, b = feature_prep(g["q_raw"], g["k_raw"], g["beta_logit"])
    o2, S2 = chunk_fwd(qh, kh, g["v"], b, g["S0"], C, alpha=alpha)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_chunk_fwd_features_empty_sequence(gpu_lib):
    w = I.ChunkWorkload("empty", 1, 2, 0, 64, 64, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_raw_inputs(w, seed=1)
    g = {k: t.to(DEV) for k, t in x.items()}
    o, S = chunk_fwd(g["q_raw"], g["k_raw"], g["v"], g["beta_logit"], g["S0"], 64, features=True)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(S, g["S0"])


def test_chunk_fwd_features_long_context(gpu_lib):
    """L = 65536, 32 heads of d = 128, C = 128 at full size from raw
    projections, o stored in fp32 and in bf16; every head against the oracle
    (the oracle's feature maps, then its forward)."""
    w = I.WORKLOADS[3]
    _note(f"[features] chunk {w.name}")
    x = I.make_chunk_raw_inputs(w, seed=0)
    g = {k: (None if t is None else t.to(DEV)) for k, t in x.items()}
    outs = []
    for od in (torch.float32, torch.bfloat16):
        o, S = chunk_fwd(g["q_raw"], g["k_raw"], g["v"], g["beta_logit"], None, w.C,
                         out_dtype=od, features=True)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(S).all()
        outs.append((o.cpu(), S.cpu()))
    del g
    (o32, S), (o16, S16) = outs
    assert torch.equal(S, S16)
    _note(f"  oracle on all {w.B * w.H} heads")
    o_ref, S_ref = oracle_heads(features_forward,
                                (x["q_raw"], x["k_raw"], x["v"], x["beta_logit"], x["S0"], None),
                                dtype="bf16")
    e = assert_parity(o32, o_ref, "bf16", "o")
    eS = assert_parity(S, S_ref, "bf16", "S_final")
    e16, floor = check_bf16_out(o16, o32, o_ref, e)
    wh = worst_head(o32, o_ref)
    _note(f"  o err/RMS = {e:.3e} (worst head {wh}), bf16 out {e16:.3e} (rounding floor "
          f"{floor:.3e}), S_final {eS:.3e}")
    record("features_workload3", workload=w.name + "_features", heads=w.B * w.H,
           o_f32_out=e, o_bf16_out=e16, bf16_rounding_floor=floor, S_final=eS,
           worst_head_f32_out=wh)


@pytest.mark.parametrize("dt,dk,dv,gated", [("bf16", 128, 128, False), ("bf16", 64, 128, True),
                                            ("f32", 128, 64, False), ("f32", 64, 64, True)])
def test_decode_features_parity(gpu_lib, dt, dk, dv, gated):
    """Eight steps in a row, the state carried; each step's inputs are raw."""
    w = I.DecodeWorkload("dec", 3, 5, dk, dv, 8, dt, 0.1)
    _note(f"[features] decode {dt} {dk}x{dv} gated={gated}")
    S = I.make_decode_state(w, seed=4)
    S_dev = S.to(DEV)
    S_ref = to64(S)
    for step in range(w.steps):
        x = I.make_decode_raw_step_inputs(w, step, seed=4)
        alpha = I.make_decode_alpha(w, step, seed=4) if gated else None
        g = {k: t.to(DEV) for k, t in x.items()}
        o = decode_step(g["q_raw"], g["k_raw"], g["v"], g["beta_logit"], S_dev,
                        alpha=None if alpha is None else alpha.to(DEV), features=True)
        qh, kh, b = feature_maps(to64(x["q_raw"]), to64(x["k_raw"]), to64(x["beta_logit"]), dt)
        if gated:
            o_ref, S_ref = gated_delta_rule_decode_step(qh, kh, to64(x["v"]), to64(alpha), b, S_ref)
        else:
            o_ref, S_ref = delta_rule_decode_step(qh, kh, to64(x["v"]), b, S_ref)
        torch.cuda.synchronize()
        assert_parity(o.cpu(), o_ref, dt, f"step {step} o")
    assert_parity(S_dev.cpu(), S_ref, dt, "S after 8 steps")


def test_decode_features_match_chunk_features(gpu_lib):
    """T fused decode steps from S0 and one fused chunked forward over the
    same T tokens reach the same outputs and state."""
    B, H, T, d = 2, 3, 40, 128
    w = I.ChunkWorkload("dvc", B, H, T, d, d, 64, "bf16", s0_std=0.1)
    x = I.make_chunk_raw_inputs(w, seed=6)
    g = {k: t.to(DEV) for k, t in x.items()}
    o_c, S_c = chunk_fwd(g["q_raw"], g["k_raw"], g["v"], g["beta_logit"], g["S0"], 64,
                         features=True)
    S = g["S0"].clone()
    outs = []
    for t in range(T):
        outs.append(decode_step(g["q_raw"][:, :, t].contiguous(), g["k_raw"][:, :, t].contiguous(),
                                g["v"][:, :, t].contiguous(), g["beta_logit"][:, :, t].contiguous(),
                                S, features=True))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=2)
    assert_parity(o_d.cpu(), to64(o_c.cpu()), "bf16", "decode vs chunk o")
    assert_parity(S.cpu(), to64(S_c.cpu()), "bf16", "decode vs chunk S")
