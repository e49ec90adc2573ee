"""The parallel head-group runner returns what the oracle returns on the whole
tensor: every head, a subset of heads, None arguments and keyword arguments."""

import numpy as np
import torch

from oracle import delta_rule_forward, gated_delta_rule_forward, kda_delta_rule_forward
from oracle_pool import features_forward, oracle_heads


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_all_heads_equal_direct_call():
    rng = np.random.default_rng(3)
    B, H, L, dk, dv = 2, 3, 19, 8, 5
    q, k, v = _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dk), _rand(rng, B, H, L, dv)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = 1 / (1 + np.exp(-_rand(rng, B, H, L)))
    S0 = 0.1 * _rand(rng, B, H, dk, dv)
    o_ref, S_ref = delta_rule_forward(q, k, v, beta, S0)
    o, S = oracle_heads(delta_rule_forward, (q, k, v, beta, S0))
    assert o.shape == o_ref.shape and S.shape == S_ref.shape
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-13)
    o, S = oracle_heads(delta_rule_forward, (q, k, v, beta, None))
    o_ref, S_ref = delta_rule_forward(q, k, v, beta, None)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)


def test_head_subset_and_torch_bf16_inputs():
    rng = np.random.default_rng(4)
    B, H, L, d = 2, 4, 11, 8
    q = torch.from_numpy(_rand(rng, B, H, L, d)).to(torch.bfloat16)
    k = torch.from_numpy(_rand(rng, B, H, L, d)).to(torch.bfloat16)
    v = torch.from_numpy(_rand(rng, B, H, L, d)).to(torch.bfloat16)
    beta = torch.rand(B, H, L, generator=torch.Generator().manual_seed(0))
    alpha = torch.rand(B, H, L, generator=torch.Generator().manual_seed(1))
    heads = [(1, 3), (0, 0), (1, 1)]
    o, S = oracle_heads(gated_delta_rule_forward, (q, k, v, alpha, beta, None), heads)
    f64 = lambda t: t.to(torch.float64).numpy()
    o_ref, S_ref = gated_delta_rule_forward(f64(q), f64(k), f64(v), f64(alpha), f64(beta))
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    np.testing.assert_allclose(o[0], o_ref[bi, hi], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0], S_ref[bi, hi], rtol=0, atol=1e-13)


def test_kda_and_feature_forms():
    rng = np.random.default_rng(5)
    B, H, L, d = 1, 3, 9, 8
    q, k, v = _rand(rng, B, H, L, d), _rand(rng, B, H, L, d), _rand(rng, B, H, L, d)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = 1 / (1 + np.exp(-_rand(rng, B, H, L)))
    alpha = 1 / (1 + np.exp(-3 - _rand(rng, B, H, L, d)))
    o, S = oracle_heads(kda_delta_rule_forward, (q, k, v, alpha, beta, None))
    o_ref, S_ref = kda_delta_rule_forward(q, k, v, alpha, beta, None)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    o, S = oracle_heads(features_forward, (q, k, v, _rand(rng, B, H, L), None, None), dtype="f32")
    assert np.isfinite(o).all() and o.shape == (B, H, L, d)
