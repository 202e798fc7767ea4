"""Budget-constrained tree selection (float64).

jisaku.com glossary, tree-topology strategies (budget-constrained
optimisation): the tree's node count is capped (64 nodes, say) and the
branches are allotted to maximise the expected number of accepted tokens.
LLM Primer ch. 9, section 9.2: EAGLE-2 grows the draft tree dynamically and
the target picks the best of several paths.

Reading: a candidate node's chance of being accepted is estimated by the
draft itself, as the product of q along its root-to-node path, so its score
is the cumulative log q, score(i) = score(parent(i)) + log q(token(i)),
score(root) = 0. The expected accepted count of a subtree is the sum of its
non-root nodes' exp(score). Since a child never scores above its parent
(log q <= 0), the M best nodes by score (ties to the lower index, which is
the ancestor) form a subtree, and no other subtree of M nodes has a larger
sum: the budget problem is solved by taking the top M. A log q above 0 (a
rounding artefact) counts as 0.
"""

from __future__ import annotations

import numpy as np


def select_topm(parent, token, logq, M: int):
    """Keep the M best candidate nodes of each tree and renumber them.

    parent int [B, Nc] (topological: parent[0] = -1, 0 <= parent[i] < i),
    token int [B, Nc], logq float64 [B, Nc] (log q of node i's token under its
    parent's draft row; the root's entry is ignored). Returns (out_parent
    int32 [B, M], out_token int32 [B, M], out_src int32 [B, M]): the kept
    nodes in ascending original index, out_src their original indices and
    out_parent their parents' new indices. Raises ValueError on a bad tree, a
    NaN log q or M outside [1, Nc].
    """
    par = np.asarray(parent)
    tok = np.asarray(token)
    lq = np.asarray(logq, dtype=np.float64)
    B, Nc = par.shape
    if not 1 <= M <= Nc:
        raise ValueError("M must be in [1, Nc]")
    out_parent = np.empty((B, M), np.int32)
    out_token = np.empty((B, M), np.int32)
    out_src = np.empty((B, M), np.int32)
    for b in range(B):
        if par[b, 0] != -1 or any(not (0 <= par[b, i] < i) for i in range(1, Nc)):
            raise ValueError(f"oracle select: bad parent array (sequence {b})")
        if np.isnan(lq[b, 1:]).any():
            raise ValueError(f"oracle select: NaN log q (sequence {b})")
        score = [0.0] * Nc
        for i in range(1, Nc):
            score[i] = score[int(par[b, i])] + min(float(lq[b, i]), 0.0)
        best = sorted(range(Nc), key=lambda i: (-score[i], i))[:M]
        kept = sorted(best)
        new = {old: j for j, old in enumerate(kept)}
        for j, old in enumerate(kept):
            out_src[b, j] = old
            out_token[b, j] = tok[b, old]
            out_parent[b, j] = -1 if old == 0 else new[int(par[b, old])]
    return out_parent, out_token, out_src


def widths_by_entropy(entropy, w_min: int, w_max: int):
    """Entropy-based branching widths for one frontier per row.

    jisaku.com glossary, tree-topology strategies (entropy-based branching):
    a node whose draft distribution has higher entropy gets more branches.
    Reading: the frontier nodes of a row are ranked by entropy, ascending
    (the lower index first among equal entropies); the node of rank r among
    F gets w_min + floor((w_max - w_min + 1) * r / F) branches, so with
    widths 1..4 each quartile of the frontier gets one width.

    entropy float64 [B, F] -> int32 [B, F]. Raises ValueError on a NaN or
    w_min > w_max or w_min < 0.
    """
    h = np.asarray(entropy, dtype=np.float64)
    if not 0 <= w_min <= w_max:
        raise ValueError("need 0 <= w_min <= w_max")
    if np.isnan(h).any():
        raise ValueError("NaN entropy")
    B, F = h.shape
    out = np.empty((B, F), np.int32)
    span = w_max - w_min + 1
    for b in range(B):
        order = sorted(range(F), key=lambda i: (h[b, i], i))
        for r, i in enumerate(order):
            out[b, i] = w_min + (span * r) // F
    return out
