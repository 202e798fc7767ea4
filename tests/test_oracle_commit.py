"""Pins for the oracle's KV commit (CPU only).

The oracle writes accepted rows through the block table. The pin reads them
back through an inverse map built from the table (physical block -> sequence,
logical block), checks every committed row against the tree row it came from,
and checks that every other byte of both caches is unchanged.
"""

import numpy as np
import pytest

import oracle
from synth import make_workload


def _inverse_map(table, nblk):
    inv = {}
    for b in range(table.shape[0]):
        for j in range(table.shape[1]):
            if table[b, j] >= 0:
                inv[int(table[b, j])] = (b, j)
    return inv


@pytest.mark.parametrize("seed,N,L", [(0, 5, (128, 128)), (1, 40, (17, 60)), (2, 64, (0, 31))])
def test_commit_writes_exactly_the_path(seed, N, L):
    w = make_workload("tiny", N=N, L=L, B=3, tree="random", with_logits=False, seed=seed)
    rng = np.random.default_rng(seed)
    path = np.full((w.B, N), -1, np.int32)
    n_acc = np.zeros(w.B, np.int32)
    for b in range(w.B):        # any root-down chain of the tree
        u, p = 0, [0]
        while True:
            kids = [c for c in range(N) if w.parent[b, c] == u]
            if not kids or rng.random() < 0.2:
                break
            u = int(rng.choice(kids))
            p.append(u)
        path[b, :len(p)] = p
        n_acc[b] = len(p) - 1
    k2, v2, slots, new_len = oracle.kv_commit(w.k_tree, w.v_tree, path, n_acc, w.block_table,
                                              w.prefix_len, w.k_cache, w.v_cache)
    inv = _inverse_map(w.block_table, w.k_cache.shape[0])
    touched = np.zeros(w.k_cache.shape[:1] + (w.block,), bool)
    for b in range(w.B):
        assert new_len[b] == w.prefix_len[b] + n_acc[b] + 1
        for t in range(N):
            if t > n_acc[b]:
                assert slots[b, t] == -1
                continue
            blk, s = divmod(int(slots[b, t]), w.block)
            assert inv[blk] == (b, (int(w.prefix_len[b]) + t) // w.block)
            assert s == (int(w.prefix_len[b]) + t) % w.block
            node = path[b, t]
            np.testing.assert_array_equal(k2[blk, :, s, :], w.k_tree[b, node])
            np.testing.assert_array_equal(v2[blk, :, :, s], w.v_tree[b, node])
            touched[blk, s] = True
    # everything else unchanged, bit for bit
    kt = np.broadcast_to(touched[:, None, :, None], k2.shape)
    vt = np.broadcast_to(touched[:, None, None, :], v2.shape)
    np.testing.assert_array_equal(k2[~kt], w.k_cache[~kt])
    np.testing.assert_array_equal(v2[~vt], w.v_cache[~vt])


def test_commit_rejects_short_block_table():
    w = make_workload("tiny", N=5, L=(128, 128), with_logits=False, seed=0)
    table = w.block_table[:, :8].copy()            # 8 blocks = 128 tokens, no room
    path = np.array([[0, 1, -1, -1, -1]], np.int32)
    with pytest.raises(ValueError):
        oracle.kv_commit(w.k_tree, w.v_tree, path, np.array([1], np.int32), table,
                         w.prefix_len, w.k_cache, w.v_cache)
