"""Tree expansion from draft rows: top-k tokens, their log-probabilities and
the row's entropy (float64).

jisaku.com glossary, tree-topology strategies: top-k branching expands each
node's k most likely draft tokens (k shrinking with depth); entropy-based
branching gives a node more branches the higher the entropy of its draft
distribution. Both read, per frontier node, q = softmax(draft row / T), its
k most likely tokens and H(q).
"""

from __future__ import annotations

import numpy as np

from .sampling import softmax


def expand_topk(draft_logits, k: int, temperature: float = 1.0):
    """Returns (top_token int32 [R, k], top_logq float64 [R, k], entropy float64 [R]).

    draft_logits float32 [R, V]. top_token[r] are the k tokens of largest
    q = softmax(row / T), in decreasing order, the lower token first among
    equal logits; top_logq = log q of those tokens; entropy = -sum q log q
    over the tokens with q > 0. Raises ValueError on a row with a NaN or no
    finite maximum, or k outside [1, V].
    """
    x = np.asarray(draft_logits, dtype=np.float32)
    R, V = x.shape
    if not 1 <= k <= V:
        raise ValueError("k must be in [1, V]")
    tok = np.empty((R, k), np.int32)
    logq = np.empty((R, k), np.float64)
    ent = np.empty(R, np.float64)
    for r in range(R):
        row = x[r]
        if np.isnan(row).any() or not np.isfinite(row.max()):
            raise ValueError(f"oracle expand: non-finite logits (row {r})")
        order = np.argsort(-row.astype(np.float64), kind="stable")   # ties: lower token first
        q = softmax(row, temperature)
        tok[r] = order[:k]
        with np.errstate(divide="ignore"):
            logq[r] = np.log(q[order[:k]])
        nz = q > 0
        ent[r] = float(-(q[nz] * np.log(q[nz])).sum())
    return tok, logq, ent
