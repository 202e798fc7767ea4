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


SPLITMIX_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(state):
    """SplitMix64 output for each uint64 state (the state after its Weyl
    increment): Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators" (OOPSLA 2014), with the finalizer of Vigna's reference code:
    z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27, z *= 0x94D049BB133111EB,
    z ^= z >> 31 (arithmetic mod 2^64)."""
    z = np.asarray(state, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def gumbel_uniforms(R: int, V: int, seed: int, offset: int):
    """float64 [R, V] uniforms of the sampling keys: u = fl64(m + 1/2) 2^-53
    with the 53-bit integer m = hi 2^21 + lo.

    hi (32 bits) of token t in row r: SplitMix64 seeded with K, output number
    r 2^20 + t div 2 + 1, i.e. the finalizer of K + (r 2^20 + t div 2 + 1) gamma,
    taking its high half for even t and its low half for odd t; K is word 0 of
    Philox4x64-10 at counter (offset, 0, 0, 3) under key (seed, 0).
    lo (21 bits): the top 21 bits of 32-bit half (t mod 8) div 4 (0: high,
    1: low) of word (t mod 8) mod 4 of Philox4x64-10 at counter
    (offset, r, t div 8, 2) under key (seed, 0).
    The walk's node uniforms use counter word 3 = 0, so no stream meets them.
    """
    from .sampling import philox4x64_10
    K = philox4x64_10(np.array([[offset, 0, 0, 3]], np.uint64), (seed, 0))[0, 0]
    idx = (np.arange(R, dtype=np.uint64)[:, None] << np.uint64(20)) + \
        (np.arange(V, dtype=np.uint64)[None, :] >> np.uint64(1)) + np.uint64(1)
    with np.errstate(over="ignore"):
        z = splitmix64(K + idx * np.uint64(SPLITMIX_GAMMA))
    odd = (np.arange(V) & 1).astype(bool)[None, :]
    hi = np.where(odd, z & np.uint64(0xFFFFFFFF), z >> np.uint64(32))

    nb = (V + 7) // 8
    ctr = np.zeros((R, nb, 4), np.uint64)
    ctr[:, :, 0] = np.uint64(offset)
    ctr[:, :, 1] = np.arange(R, dtype=np.uint64)[:, None]
    ctr[:, :, 2] = np.arange(nb, dtype=np.uint64)[None, :]
    ctr[:, :, 3] = np.uint64(2)
    w = philox4x64_10(ctr.reshape(-1, 4), (seed, 0)).reshape(R, nb, 4)
    halves = np.empty((R, nb, 8), np.uint64)
    halves[:, :, :4] = w >> np.uint64(32)                   # tokens 8j .. 8j+3
    halves[:, :, 4:] = w & np.uint64(0xFFFFFFFF)            # tokens 8j+4 .. 8j+7
    lo = halves.reshape(R, nb * 8)[:, :V] >> np.uint64(11)
    m = (hi << np.uint64(21)) | lo
    return (m.astype(np.float64) + 0.5) * 2.0 ** -53


def gumbel_keys(draft_logits, temperature: float, seed: int, offset: int):
    """float64 [R, V] sampling keys x/T + G, G = -log(-log u) a standard
    Gumbel draw from ``gumbel_uniforms``; x/T and the sum in float64."""
    x = np.asarray(draft_logits, dtype=np.float32)
    R, V = x.shape
    u = gumbel_uniforms(R, V, seed, offset)
    g = -np.log(-np.log(u))
    with np.errstate(invalid="ignore"):
        return x.astype(np.float64) / float(temperature) + g


def expand_sample(draft_logits, k: int, temperature: float, seed: int, offset: int):
    """k children per row drawn from q = softmax(row / T) without replacement.

    Reading of the glossary's top-k branching for a sampled tree: ranking a
    row by x/T plus independent Gumbel noise and keeping the k largest is a
    draw of k tokens from q without replacement, largest key first being the
    order of sequential draws (the Gumbel-top-k construction). Keys are
    those of ``gumbel_keys`` (float64); the lower token first among equal
    keys.
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
    order = np.argsort(-keys, axis=1, kind="stable")   # ties: lower token
    tok = order[:, :k].astype(np.int32)
    q = softmax(x, temperature)
    with np.errstate(divide="ignore"):
        logq = np.log(np.take_along_axis(q, tok.astype(np.int64), axis=1))
        plogp = np.where(q > 0, q * np.log(np.where(q > 0, q, 1.0)), 0.0)
    ent = -plogp.sum(axis=1)
    return tok, logq, ent
