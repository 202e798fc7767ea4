"""GPU parity of tree_topology_dp (the budget's best topology under
acceptance by sibling rank) against the oracle's program: bit-exact parents,
ranks and value (both sides form every value with the same fp64 operations
in the same order and break ties alike)."""

import numpy as np
import pytest
import torch

import tree_attention_verification_ancestor_amd as tav
from oracle.topology import topology
from synth.device import to_numpy

from gpu_helpers import device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,n,depth,seed", [
    (4, 64, 6, 0), (4, 128, 8, 1), (3, 16, 4, 2), (1, 6, 5, 3), (16, 64, 10, 4),
    (5, 150, 3, 5), (2, 1, 0, 6), (4, 5, 1, 7), (8, 256, 8, 8),
])
def test_topology_matches_oracle(K, n, depth, seed):
    say(f"topology dp: K={K} n={n} depth={depth}")
    rng = np.random.default_rng(seed)
    p = np.sort(rng.uniform(0.05, 0.95, K))[::-1]
    if seed % 3 == 0:
        p = rng.uniform(0.0, 1.0, K)          # unsorted rates too
    parent, rank, value = tav.tree_topology_dp(list(p), n, depth, device=device())
    torch.cuda.synchronize()
    rp, rr, rv = topology(p, n, depth)
    np.testing.assert_array_equal(to_numpy(parent), rp)
    np.testing.assert_array_equal(to_numpy(rank), rr)
    assert to_numpy(value)[0] == rv
