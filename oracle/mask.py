"""Tree attention mask, the plain definition.

jisaku.com glossary "Tree-based speculative decoding", section on how tree
attention works: entry M[i][j] is 1 exactly when node j lies on the path from
the root to node i (node i included), and 0 otherwise. The radar-34b blog,
section 3 ("Tree Attention Verification Matrix"), prints the 5-node instance.

Packing (a reading; the pages fix none): word ``j // 64``, bit ``j % 64`` of
row i holds M[i][j]; unused high bits are zero.
"""

from __future__ import annotations

import numpy as np


def _check_parent(parent_row: np.ndarray) -> None:
    n = parent_row.shape[0]
    if n < 1:
        raise ValueError("empty tree")
    if int(parent_row[0]) != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    for i in range(1, n):
        p = int(parent_row[i])
        if not (0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is not an earlier node")


def ancestor_matrix(parent_row: np.ndarray) -> np.ndarray:
    """Boolean M[i][j]: j is node i or one of its ancestors."""
    parent_row = np.asarray(parent_row)
    _check_parent(parent_row)
    n = parent_row.shape[0]
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j != -1:          # climb to the root, marking every node met
            m[i, j] = True
            j = int(parent_row[j])
    return m


def tree_mask(parent: np.ndarray):
    """Packed ancestor-or-self masks and depths for a batch of trees.

    parent: int [B, N].  Returns (mask uint64 [B, N, ceil(N/64)], depth int32 [B, N]).
    Raises ValueError for a row that is not a rooted tree in topological order.
    """
    parent = np.asarray(parent)
    B, N = parent.shape
    W = (N + 63) // 64
    mask = np.zeros((B, N, W), dtype=np.uint64)
    depth = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        m = ancestor_matrix(parent[b])
        for i in range(N):
            for j in np.nonzero(m[i])[0]:
                mask[b, i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
            depth[b, i] = int(m[i].sum()) - 1     # ancestors other than itself
    return mask, depth
