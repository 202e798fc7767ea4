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


def gumbel_keys(draft_logits, temperature: float, seed: int, offset: int):
    """float32 [R, V] sampling keys: y + G with y = x * (1/T) and G a standard
    Gumbel draw, both rounded to float32 and added in float32.

    G = -log(-log u) with u = ((w >> 11) + 1/2) * 2^-53 from Philox4x64-10
    word (token mod 4) at counter (offset, row, token div 4, 1) under key
    (seed, 0); the walk's node uniforms use counter word 3 = 0, so the two
    streams never meet.
    """
    from .sampling import philox4x64_10
    x = np.asarray(draft_logits, dtype=np.float32)
    R, V = x.shape
    invT = np.float32(1.0 / float(temperature))
    nq = (V + 3) // 4
    ctr = np.zeros((R, nq, 4), np.uint64)
    ctr[:, :, 0] = np.uint64(offset)
    ctr[:, :, 1] = np.arange(R, dtype=np.uint64)[:, None]
    ctr[:, :, 2] = np.arange(nq, dtype=np.uint64)[None, :]
    ctr[:, :, 3] = np.uint64(1)
    w = philox4x64_10(ctr.reshape(-1, 4), (seed, 0)).reshape(R, nq * 4)[:, :V]
    u = ((w >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    g = -np.log(-np.log(u))
    return (x * invT).astype(np.float32) + g.astype(np.float32)


def expand_sample(draft_logits, k: int, temperature: float, seed: int, offset: int):
    """k children per row drawn from q = softmax(row / T) without replacement.

    Reading of the glossary's top-k branching for a sampled tree: ranking a
    row by x/T plus independent Gumbel noise and keeping the k largest is a
    draw of k tokens from q without replacement, largest key first being the
    order of sequential draws (the Gumbel-top-k construction). Keys are
    those of ``gumbel_keys``; the lower token first among equal keys.
    Returns (token int32 [R, k], log q float64 [R, k], entropy float64 [R])
    with log q and the entropy as in ``expand_topk``. Raises ValueError as
    ``expand_topk`` does.
    """
    x = np.asarray(draft_logits, dtype=np.float32)
    R, V = x.shape
    if not 1 <= k <= V:
        raise ValueError("k must be in [1, V]")
    keys = gumbel_keys(x, temperature, seed, offset)
    if np.isnan(x).any() or not np.isfinite(x.max(axis=1)).all():
        bad = int(np.nonzero(np.isnan(x).any(axis=1) | ~np.isfinite(x.max(axis=1)))[0][0])
        raise ValueError(f"oracle expand: non-finite logits (row {bad})")
    order = np.argsort(-keys.astype(np.float64), axis=1, kind="stable")   # ties: lower token
    tok = order[:, :k].astype(np.int32)
    q = softmax(x, temperature)
    with np.errstate(divide="ignore"):
        logq = np.log(np.take_along_axis(q, tok.astype(np.int64), axis=1))
        plogp = np.where(q > 0, q * np.log(np.where(q > 0, q, 1.0)), 0.0)
    ent = -plogp.sum(axis=1)
    return tok, logq, ent
