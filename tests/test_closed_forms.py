"""Closed-form references that GPU tests use at sizes the oracle cannot reach, checked here against
the fp64 oracle on small instances of the same structured inputs."""
import numpy as np
import pytest

from oracle import attn_oracle
from tests.test_large_gpu import A_CLS, B_STAR, long_reference


@pytest.mark.parametrize("n_keys,k_star", [(1000, [500, 999]), (7 * 37, [0, 7 * 37 - 1]), (129, [64, 3])])
def test_long_reference_matches_oracle(n_keys, k_star):
    d, sq = 16, 6
    jj = np.arange(d, dtype=np.float64)
    base = np.stack([((jj + 3 * c) % 7 - 3) / 4 for c in range(7)])
    v_star = ((jj % 5) - 2) / 2
    r = np.arange(n_keys) % 7
    k = np.zeros((1, 2, n_keys, d))
    v = np.zeros((1, 2, n_keys, d))
    for h in range(2):
        k[0, h, :, 0] = np.array(A_CLS)[r]
        k[0, h, k_star[h], 0] = B_STAR
        v[0, h] = base[r]
        v[0, h, k_star[h]] = v_star
    q = np.zeros((1, 2, sq, d))
    q[0, :, 0::2, 0] = 1.0
    q[0, :, 1::2, 0] = 0.5
    o, lse = attn_oracle.get().attention(q, k, v, False, 1.0)
    ro, rl = long_reference(k_star, base, v_star, n_keys=n_keys, sq=sq)
    assert np.abs(o[0] - ro).max() < 1e-12
    assert np.abs(lse[0] - rl).max() < 1e-12
