"""Budget-constrained tree topology by dynamic programming (float64).

jisaku.com glossary, tree-topology strategies (budget-constrained
optimisation): the node count is capped and branches are allotted to
maximise the expected number of accepted tokens, a problem solved by dynamic
programming; the Sequoia paragraph of the same page has the topology chosen
for the hardware and made robust to how the draft behaves.

Reading (the acceptance model is not given on the pages): acceptance by
sibling rank. The k-th child of any node (k = 1, 2, ..., in the order the
walk tries siblings) is accepted with probability p_k once the walk has
reached its parent and rejected its k - 1 earlier siblings, the same p_k at
every depth. A node is reached, and accepted, with the product of the p of
the ranks along its root-to-node path, so the expected accepted count of a
tree is the sum over its non-root nodes of those path products. With every
p_k = 0 beyond k = 1 the optimum is the chain, whose value is the closed form
sum_{i=1}^{n-1} p_1^i.

The program, for a subtree of m nodes whose root may have descendants r
levels below it:
    F(1, r) = 0;  F(m, 0) = -inf for m > 1;
    F(m, r) = C(m - 1, r - 1, 1),
    C(0, r, j) = 0;  C(s, r, j) = -inf if j > K;
    C(s, r, j) = max over t = 1..s of  p_j (1 + F(t, r)) + C(s - t, r, j + 1),
where C(s, r, j) places s nodes in the subtrees of children j, j + 1, ...
(each subtree s >= 1 nodes deep at most r). Every value is formed in that
order in float64 (a = 1 + F; b = p_j * a; b + C), and among equal maxima the
smallest t wins. The tree is written out breadth-first: node 0 the root,
then each node's children in rank order, appended as they are reached.
"""

from __future__ import annotations

import math

import numpy as np

NEG = -math.inf


def dp_tables(p, n: int, depth: int):
    """F[r][m] (m = 0..n, r = 0..depth) and the argmax child sizes
    T[r][j][s] of C(s, r, j) (r = 0..depth-1, j = 1..K, s = 1..n-1)."""
    p = [float(x) for x in p]
    K = len(p)
    F = [[NEG] * (n + 1) for _ in range(depth + 1)]
    T = [[[0] * n for _ in range(K + 2)] for _ in range(depth)]
    for r in range(depth + 1):
        F[r][1] = 0.0
    for r in range(1, depth + 1):
        rr = r - 1                      # the children's subtrees may go rr deeper
        # C over j = K..1 for s = 0..n-1
        C_next = [0.0] + [NEG] * (n - 1)          # j = K + 1: only s = 0
        for j in range(K, 0, -1):
            C = [0.0] + [NEG] * (n - 1)
            for s in range(1, n):
                best, arg = NEG, 0
                for t in range(1, s + 1):
                    f = F[rr][t]
                    rest = C_next[s - t]
                    if f == NEG or rest == NEG:
                        continue
                    a = 1.0 + f
                    b = p[j - 1] * a
                    v = b + rest
                    if v > best:
                        best, arg = v, t
                C[s] = best
                T[rr][j][s] = arg
            C_next = C
        for m in range(2, n + 1):
            F[r][m] = C_next[m - 1]
    return F, T


def topology(p, n: int, depth: int):
    """The n-node tree of depth at most `depth` with the largest expected
    accepted count under sibling-rank acceptance p[0..K-1] (see the module).

    Returns (parent int32 [n], rank int32 [n] (1-based position among its
    siblings, 0 for the root), value float64). Raises ValueError for n < 1,
    depth < 0, p outside [0, 1] or NaN, or no tree of n nodes within the
    depth and K children per node.
    """
    p = [float(x) for x in p]
    if n < 1 or depth < 0 or not p or any(not (0.0 <= x <= 1.0) for x in p):
        raise ValueError("bad arguments")
    K = len(p)
    F, T = dp_tables(p, n, depth)
    if F[depth][n] == NEG:
        raise ValueError("no tree of that size fits the depth and width limits")
    parent = [-1]
    rank = [0]
    queue = [(0, n, depth)]           # (node, subtree size, levels left)
    head = 0
    while head < len(queue):
        node, m, r = queue[head]
        head += 1
        s, j = m - 1, 1
        while s > 0:
            t = T[r - 1][j][s]
            parent.append(node)
            rank.append(j)
            queue.append((len(parent) - 1, t, r - 1))
            s -= t
            j += 1
    return (np.array(parent, np.int32), np.array(rank, np.int32), float(F[depth][n]))


def tree_value(parent, rank, p) -> float:
    """Expected accepted count of a tree under sibling-rank acceptance: the
    sum over non-root nodes of the product of p[rank - 1] along the path."""
    n = len(parent)
    prod = [1.0] * n
    total = 0.0
    for i in range(1, n):
        prod[i] = prod[int(parent[i])] * float(p[int(rank[i]) - 1])
        total += prod[i]
    return total
