"""The chunked backward the HIP kernels implement (wy_model.chunked_backward,
fp64) against the backward oracle, for several chunk sizes and ragged
tails: the chunk-level algebra is exact."""

import numpy as np
import pytest

from oracle import delta_rule_backward
from wy_model import chunked_backward


@pytest.mark.parametrize("C", [1, 7, 16, 64])
@pytest.mark.parametrize("with_states", [True, False])
def test_chunked_backward_matches_oracle(C, with_states):
    rng = np.random.default_rng(3 + C)
    B, H, L, dk, dv = 1, 2, 45, 6, 5
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, L, dv))
    beta = rng.uniform(0, 1, (B, H, L))
    dO = rng.standard_normal((B, H, L, dv))
    S0 = rng.standard_normal((B, H, dk, dv)) if with_states else None
    dSf = rng.standard_normal((B, H, dk, dv)) if with_states else None
    ref = delta_rule_backward(q, k, v, beta, S0, dO, dSf)
    got = chunked_backward(q, k, v, beta, S0, dO, dSf, C)
    for name, a, b in zip(("dq", "dk", "dv", "dbeta", "dS0"), got, ref):
        assert np.abs(a - b).max() < 1e-12, name
