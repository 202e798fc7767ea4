"""Exact losslessness of the oracle's walk on small vocabularies (CPU).

radar-34b blog §2 (rejection-sampling acceptance condition): a draft x from q
is kept with probability min(1, p(x)/q(x)); after a rejection the next draw
comes from the normalised positive part of p - q. Its proof sketch claims
that the emitted token then follows p exactly. This test computes, with
rational arithmetic, the distribution of the first token the oracle's walk
emits at a root with k children, and requires it to equal p as a fraction.

How it stays exact without retyping the rule: p and q are rationals a_y / D
(logits log a_y, so the oracle's fp64 softmax gives them to ~1e-7); the
children's tokens are enumerated with their draft probabilities (independent
draws from q, or sequential draws without replacement); every uniform the
walk can read (each child's acceptance uniform and the root's resampling
uniform) runs over the M midpoints (i + 1/2)/M of a grid, through the
oracle's own code (uniforms passed in). M is a common denominator of every
boundary the rule meets for that p and q (found once, offline, by exact
enumeration of the walk's residuals), so each midpoint is at least 1/(2M)
from every boundary and the fraction of grid points with an outcome is that
outcome's exact probability.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _first_token_distribution(a, b, k, M, wor):
    V = len(a)
    D = sum(a)
    assert sum(b) == D
    p = [Fraction(x, D) for x in a]
    q = [Fraction(x, D) for x in b]
    tl = np.log(np.array(a, np.float64)).astype(np.float32)
    dl = np.log(np.array(b, np.float64)).astype(np.float32)
    N = k + 1
    parent = np.array([-1] + [0] * k, np.int32)
    grid = (np.arange(M, dtype=np.float64) + 0.5) / M
    # every combination of the k acceptance uniforms and the root's resampling one
    G = M ** (k + 1)
    idx = np.indices((M,) * (k + 1)).reshape(k + 1, G)
    u = np.zeros((G, N, 2))
    u[:, 0, 1] = grid[idx[0]]
    for c in range(1, N):
        u[:, c, 0] = grid[idx[c]]
        u[:, c, 1] = 0.5 / M   # a bonus draw after an accepted child: a midpoint too
    got = [Fraction(0)] * V
    tuples = itertools.permutations(range(V), k) if wor else itertools.product(range(V), repeat=k)
    for toks in tuples:
        # probability of drawing these children's tokens
        w, left = Fraction(1), Fraction(1)
        for x in toks:
            w *= q[x] / left
            if wor:
                left -= q[x]
        token = np.array([0] + list(toks), np.int32)
        res = oracle.verify_walk(np.broadcast_to(tl, (G, N, V)), np.broadcast_to(dl, (G, N, V)),
                                 np.broadcast_to(parent, (G, N)), np.broadcast_to(token, (G, N)),
                                 1.0, without_replacement=wor, uniforms=u)
        counts = np.bincount(res.out_tokens[:, 0], minlength=V)
        assert counts.sum() == G
        # no draw of the grid sits near a boundary
        assert (res.min_margin >= 1.0 / (2 * M) - 1e-6).all()
        for y in range(V):
            got[y] += w * Fraction(int(counts[y]), G)
    return p, got


@pytest.mark.parametrize("k", [1, 2, 3])
def test_independent_siblings_emit_p_exactly(k):
    # p = (1, 2, 3)/6, q = (3, 1, 2)/6: four distinct residuals within three
    # rejections; every boundary is a multiple of 1/6
    p, got = _first_token_distribution((1, 2, 3), (3, 1, 2), k, 6, wor=False)
    assert got == p


@pytest.mark.parametrize("k", [1, 2])
def test_siblings_without_replacement_emit_p_exactly(k):
    # p = (1, 2, 4, 5)/12, q = (3, 1, 6, 2)/12 under the without-replacement
    # rule: five distinct residuals; every boundary is a multiple of 1/24
    p, got = _first_token_distribution((1, 2, 4, 5), (3, 1, 6, 2), k, 24, wor=True)
    assert got == p


def test_the_exact_check_catches_the_wrong_rule():
    """Siblings drawn without replacement but tested with the independent-
    sibling rule: the same exact computation then misses p (so the check has
    the power to fail)."""
    V, D, M, k = 4, 12, 36, 2   # every boundary of the independent rule here: multiples of 1/36
    a, b = (1, 2, 4, 5), (3, 1, 6, 2)
    p = [Fraction(x, D) for x in a]
    q = [Fraction(x, D) for x in b]
    tl = np.log(np.array(a, np.float64)).astype(np.float32)
    dl = np.log(np.array(b, np.float64)).astype(np.float32)
    grid = (np.arange(M) + 0.5) / M
    G = M ** (k + 1)
    idx = np.indices((M,) * (k + 1)).reshape(k + 1, G)
    u = np.zeros((G, k + 1, 2))
    u[:, 0, 1] = grid[idx[0]]
    for c in range(1, k + 1):
        u[:, c, 0] = grid[idx[c]]
        u[:, c, 1] = 0.5 / M   # a bonus draw after an accepted child: a midpoint too
    wrong = [Fraction(0)] * V
    for toks in itertools.permutations(range(V), k):
        w = q[toks[0]] * q[toks[1]] / (1 - q[toks[0]])
        res = oracle.verify_walk(np.broadcast_to(tl, (G, k + 1, V)),
                                 np.broadcast_to(dl, (G, k + 1, V)),
                                 np.broadcast_to(np.array([-1, 0, 0], np.int32), (G, k + 1)),
                                 np.broadcast_to(np.array([0, *toks], np.int32), (G, k + 1)),
                                 1.0, uniforms=u)
        counts = np.bincount(res.out_tokens[:, 0], minlength=V)
        assert (res.min_margin >= 1.0 / (2 * M) - 1e-6).all()   # the counts are exact here too
        for y in range(V):
            wrong[y] += w * Fraction(int(counts[y]), G)
    assert sum(wrong) == 1
    assert wrong != p
    assert max(abs(float(wrong[y] - p[y])) for y in range(V)) > 1e-3
