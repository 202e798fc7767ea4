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


def _random_paths(w, rng, stop=0.2):
    N = w.N
    path = np.full((w.B, N), -1, np.int32)
    n_acc = np.zeros(w.B, np.int32)
    for b in range(w.B):
        u, p = 0, [0]
        while True:
            kids = [c for c in range(N) if w.parent[b, c] == u]
            if not kids or rng.random() < stop:
                break
            u = int(rng.choice(kids))
            p.append(u)
        path[b, :len(p)] = p
        n_acc[b] = len(p) - 1
    return path, n_acc


def _tree_in_cache(w):
    """The tree's rows written at positions L..L+N-1 by the pinned kv_commit
    (identity path)."""
    ident = np.tile(np.arange(w.N, dtype=np.int32), (w.B, 1))
    full = np.full(w.B, w.N - 1, np.int32)
    k, v, _, _ = oracle.kv_commit(w.k_tree, w.v_tree, ident, full, w.block_table, w.prefix_len,
                                  w.k_cache, w.v_cache)
    return k, v


@pytest.mark.parametrize("seed,N,L", [(3, 5, (128, 128)), (4, 40, (17, 60)), (5, 64, (0, 31)),
                                      (6, 200, (1, 300))])
def test_inplace_rollback_equals_commit_from_tree_rows(seed, N, L):
    w = make_workload("tiny", N=N, L=L, B=3, tree="random", with_logits=False, seed=seed)
    path, n_acc = _random_paths(w, np.random.default_rng(seed))
    k_tree_c, v_tree_c = _tree_in_cache(w)
    k1, v1, s1, l1 = oracle.kv_commit_inplace(path, n_acc, w.block_table, w.prefix_len,
                                              k_tree_c, v_tree_c)
    k2, v2, s2, l2 = oracle.kv_commit(w.k_tree, w.v_tree, path, n_acc, w.block_table,
                                      w.prefix_len, w.k_cache, w.v_cache)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(l1, l2)
    # the committed positions agree; outside the tree's positions both equal
    # the original cache; the abandoned positions keep the tree's rows
    inv = _inverse_map(w.block_table, w.k_cache.shape[0])
    for blk in range(w.k_cache.shape[0]):
        for s in range(w.block):
            if blk in inv:
                b, j = inv[blk]
                pos = j * w.block + s - int(w.prefix_len[b])
            else:
                b, pos = -1, -1
            if 0 <= pos <= n_acc[b]:
                np.testing.assert_array_equal(k1[blk, :, s, :], k2[blk, :, s, :])
                np.testing.assert_array_equal(v1[blk, :, :, s], v2[blk, :, :, s])
            elif 0 <= pos < w.N:
                np.testing.assert_array_equal(k1[blk, :, s, :], k_tree_c[blk, :, s, :])
                np.testing.assert_array_equal(v1[blk, :, :, s], v_tree_c[blk, :, :, s])
            else:
                np.testing.assert_array_equal(k1[blk, :, s, :], w.k_cache[blk, :, s, :])
                np.testing.assert_array_equal(v1[blk, :, :, s], w.v_cache[blk, :, :, s])


def test_inplace_rollback_of_a_chain_from_the_root_moves_nothing():
    w = make_workload("tiny", N=12, L=(30, 90), B=4, tree="chain", with_logits=False, seed=7)
    k_c, v_c = _tree_in_cache(w)
    n_acc = np.array([0, 3, 7, 11], np.int32)
    path = np.full((w.B, w.N), -1, np.int32)
    for b in range(w.B):
        path[b, :n_acc[b] + 1] = np.arange(n_acc[b] + 1)
    k1, v1, _, l1 = oracle.kv_commit_inplace(path, n_acc, w.block_table, w.prefix_len, k_c, v_c)
    np.testing.assert_array_equal(k1, k_c)
    np.testing.assert_array_equal(v1, v_c)
    np.testing.assert_array_equal(l1, w.prefix_len + n_acc + 1)


def test_inplace_rollback_rejects_a_table_too_short_for_the_tree():
    w = make_workload("tiny", N=5, L=(126, 126), with_logits=False, seed=0)
    table = w.block_table[:, :8].copy()            # 128 tokens: the tree needs 131
    path = np.array([[0, 1, -1, -1, -1]], np.int32)
    with pytest.raises(ValueError):
        oracle.kv_commit_inplace(path, np.array([1], np.int32), table, w.prefix_len,
                                 w.k_cache, w.v_cache)
