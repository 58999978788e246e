"""The library's host-side bit-width assigner against the oracle's sweep
(bit-exact assignments; no GPU needed)."""
import os

import numpy as np
import pytest

import oracle

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sparse_message_passing_amd",
                   "libgnnmp.so")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgnnmp.so not built")
@pytest.mark.parametrize("seed", range(6))
def test_assign_bits_matches_oracle(seed):
    from sparse_message_passing_amd import gnnmp
    r = np.random.default_rng(seed)
    m = int(r.integers(1, 3000))
    d = int(r.choice([64, 100, 256]))
    beta = (r.lognormal(0.0, 2.0, m) * (r.random(m) < 0.95)).astype(np.float32)
    beta[: m // 10] = beta[0]  # ties
    for avg in (2.0, 2.5, 3.3, 4.0, 6.1, 8.0):
        got = gnnmp.gnn_assign_bits(beta, d, avg)
        ref = oracle.assign_bits_greedy(beta.astype(np.float64), d, avg)
        assert np.array_equal(got, ref), (seed, avg)


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgnnmp.so not built")
def test_assign_bits_rejects_bad_input():
    from sparse_message_passing_amd import gnnmp
    with pytest.raises(gnnmp.GnnError, match="avg_bits"):
        gnnmp.gnn_assign_bits(np.ones(3, np.float32), 8, 9.0)
    with pytest.raises(gnnmp.GnnError, match="finite"):
        gnnmp.gnn_assign_bits(np.array([1.0, np.nan], np.float32), 8, 4.0)
