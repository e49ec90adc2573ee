"""The seeded input generator: deterministic, the stated distributions, and
sliced draws equal to one big draw (CPU only)."""

import numpy as np
import torch

from deltanet_delta_rule_chunk_amd import inputs as I


def test_workload_table():
    w = I.WORKLOADS
    assert [type(x).__name__ for x in w] == ["ChunkWorkload"] * 4 + ["DecodeWorkload"]
    assert (w[3].B, w[3].H, w[3].L, w[3].d_k, w[3].C) == (1, 32, 65536, 128, 128)
    assert (w[4].B, w[4].H, w[4].d_k, w[4].steps) == (256, 32, 128, 1000)


def test_chunk_inputs_recipe():
    w = I.scaled_chunk_workload(I.WORKLOADS[2], L=96)
    a = I.make_chunk_inputs(w, seed=0)
    b = I.make_chunk_inputs(w, seed=0)
    for key in ("q", "k", "v", "beta", "S0"):
        assert torch.equal(a[key], b[key]), key
    assert a["q"].dtype == torch.bfloat16 and a["beta"].dtype == torch.float32
    assert a["q"].shape == (2, 16, 96, 128) and a["S0"].shape == (2, 16, 128, 128)
    kn = a["k"].double().norm(dim=-1)
    assert (kn - 1).abs().max() < 1e-2  # unit before the bf16 cast
    beta = a["beta"]
    assert torch.all(beta[:, :8] == 1.0)
    assert torch.all((beta[:, 8:] > 0) & (beta[:, 8:] < 1))
    assert abs(float(a["S0"].std()) - 0.1) < 0.01


def test_sliced_draw_equals_single_draw():
    w = I.scaled_chunk_workload(I.WORKLOADS[0], L=32)
    a = I.make_chunk_inputs(w, seed=3)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((w.B, w.H, 32, w.d_k))
    assert torch.equal(a["q"], torch.from_numpy(q).to(torch.float32))


def test_decode_inputs():
    w = I.WORKLOADS[4]
    w_small = I.DecodeWorkload("t", 2, 3, 8, 4, 5, "bf16", 0.1)
    s = I.make_decode_state(w_small, 0)
    assert s.shape == (2, 3, 8, 4) and s.dtype == torch.float32
    x0 = I.make_decode_step_inputs(w_small, 0)
    x1 = I.make_decode_step_inputs(w_small, 1)
    assert not torch.equal(x0["q"], x1["q"])
    assert torch.equal(x0["q"], I.make_decode_step_inputs(w_small, 0)["q"])
    assert x0["beta"].shape == (2, 3)
    assert w.dtype == "bf16"
