"""Pins for the oracle's tree mask (CPU only).

The oracle builds the mask by climbing parent pointers. Each pin below reaches
the same matrix by another route: the page's printed example, the causal mask
of a chain, or DFS entry/exit intervals (j is an ancestor-or-self of i exactly
when i's entry time falls inside j's interval).
"""

import os

import numpy as np
import pytest

import oracle
from synth import chain_parent, example_parent, random_parent

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_worked_example.txt")


def _load_golden():
    rows, parent = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# parent:"):
                parent = [int(x) for x in line.split(":")[1].split()]
            elif line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()[1:]])
    return np.array(parent, np.int32), np.array(rows, bool)


def _unpack(mask_row, n):
    return np.array([[(int(mask_row[i, j // 64]) >> (j % 64)) & 1 for j in range(n)]
                     for i in range(n)], dtype=bool)


def _dfs_ancestor_matrix(parent):
    """Ancestor-or-self relation from DFS intervals over explicit child lists."""
    n = len(parent)
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[parent[i]].append(i)
    tin, tout = [0] * n, [0] * n
    clock = 0
    stack = [(0, False)]
    while stack:
        v, done = stack.pop()
        if done:
            tout[v] = clock
            continue
        tin[v] = clock
        clock += 1
        stack.append((v, True))
        for c in reversed(kids[v]):
            stack.append((c, False))
    m = np.zeros((n, n), bool)
    for i in range(n):
        for j in range(n):
            m[i, j] = tin[j] <= tin[i] < tout[j]
    return m


def _bfs_depth(parent):
    n = len(parent)
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[parent[i]].append(i)
    depth = [0] * n
    frontier = [0]
    while frontier:
        nxt = []
        for v in frontier:
            for c in kids[v]:
                depth[c] = depth[v] + 1
                nxt.append(c)
        frontier = nxt
    return np.array(depth)


def test_worked_example_matches_page():
    parent, rows = _load_golden()
    assert (parent == example_parent()).all()
    mask, depth = oracle.tree_mask(parent[None, :])
    assert mask.shape == (1, 5, 1)
    assert (_unpack(mask[0], 5) == rows).all()
    # the same rows as packed words, bit j = column j
    assert [int(w) for w in mask[0, :, 0]] == [1, 3, 7, 9, 25]
    assert list(depth[0]) == [0, 1, 2, 1, 2]


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 130, 256])
def test_chain_gives_causal_mask(n):
    mask, depth = oracle.tree_mask(chain_parent(n)[None, :])
    assert mask.shape == (1, n, (n + 63) // 64)
    assert (_unpack(mask[0], n) == np.tril(np.ones((n, n), bool))).all()
    assert (depth[0] == np.arange(n)).all()


@pytest.mark.parametrize("seed,n", [(0, 5), (1, 40), (2, 64), (3, 100), (4, 200), (5, 256)])
def test_random_tree_matches_dfs_intervals(seed, n):
    rng = np.random.default_rng(seed)
    parents = np.stack([random_parent(rng, n) for _ in range(3)])
    mask, depth = oracle.tree_mask(parents)
    for b in range(3):
        ref = _dfs_ancestor_matrix(list(parents[b]))
        assert (_unpack(mask[b], n) == ref).all()
        assert (depth[b] == _bfs_depth(list(parents[b]))).all()
        # unused high bits of the last word stay zero
        if n % 64:
            assert (mask[b, :, -1] >> np.uint64(n % 64) == 0).all()


@pytest.mark.parametrize("bad", [[0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, -1, 0], [-1, 0, 5]])
def test_invalid_parent_rejected(bad):
    with pytest.raises(ValueError):
        oracle.tree_mask(np.array([bad], np.int32))
