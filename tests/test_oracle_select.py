"""Pins for the oracle's budget-constrained tree selection (CPU only).

The pages' budget rule (jisaku.com glossary, tree-topology strategies) fixes
the objective: under a node budget, maximise the expected number of accepted
tokens. With a node's acceptance estimated as the product of draft
probabilities along its path, that is checked here without the oracle's
cumulative sums:
  * brute force: over every subtree of M nodes of small random trees, the
    largest sum of path products of q equals the sum of the oracle's pick;
  * another route: the input generator's best-first growth (a heap that pops
    the best proposed candidate, one node at a time) keeps the same token
    paths as the oracle's top-M of the fully expanded candidate tree;
  * invariants and special cases: the pick is a subtree in topological order
    whose every node scores at least every dropped node; chains keep their
    first M nodes, a star its M - 1 likeliest children, equal scores the
    lower indices, M = Nc everything.
"""

import heapq
import itertools

import numpy as np
import pytest

import oracle
from synth import random_parent
from synth.workloads import _ranked_tokens


def _path_product(par, q, i):
    prod = 1.0
    while i != 0:
        prod *= q[i]
        i = int(par[i])
    return prod


def _subtrees(par, M):
    """Every node set of size M that holds the root and each member's parent."""
    Nc = par.shape[0]
    for rest in itertools.combinations(range(1, Nc), M - 1):
        s = {0, *rest}
        if all(int(par[i]) in s for i in rest):
            yield s


@pytest.mark.parametrize("seed", range(12))
def test_pick_maximises_expected_accepted_tokens(seed):
    rng = np.random.default_rng(seed)
    Nc = int(rng.integers(2, 10))
    par = random_parent(rng, Nc)
    q = rng.uniform(0.01, 1.0, Nc)
    logq = np.log(q)
    for M in range(1, Nc + 1):
        op, ot, src = oracle.select_topm(par[None], np.arange(Nc)[None], logq[None], M)
        got = sum(_path_product(par, q, int(i)) for i in src[0] if i != 0)
        best = max(sum(_path_product(par, q, i) for i in s if i != 0) for s in _subtrees(par, M))
        assert got == pytest.approx(best, rel=1e-12, abs=1e-300)


def _full_expansion(draft_rows_of, widths, root_token):
    """Every candidate of a width-by-depth top-k expansion, level order.
    Returns parent, token, logit gap to the row maximum (the generator's
    score increment) and each node's token path."""
    parent, token, gap, path = [-1], [root_token], [0.0], [()]
    depth = [0]
    i = 0
    while i < len(parent):
        d = depth[i]
        if d < len(widths):
            row = draft_rows_of(path[i])
            mx = float(row.max())
            for x in _ranked_tokens(row, widths[d]):
                parent.append(i)
                token.append(int(x))
                gap.append(float(row[x]) - mx)
                path.append(path[i] + (int(x),))
                depth.append(d + 1)
        i += 1
    return np.array(parent), np.array(token), np.array(gap), path


def _grow_best_first(row_of, widths, budget, root_token):
    """Grow a tree one node at a time: every node proposes the top
    widths[depth] tokens of its row; the best proposal so far (largest
    cumulative logit gap, earliest proposal on ties) becomes the next node.
    Returns the token paths of the grown nodes."""
    paths, score = [()], [0.0]
    heap, seq = [], 0

    def propose(u):
        nonlocal seq
        d = len(paths[u])
        if d >= len(widths):
            return
        row = row_of(paths[u])
        mx = float(row.max())
        for x in _ranked_tokens(row, widths[d]):
            heapq.heappush(heap, (-(score[u] + (float(row[x]) - mx)), seq, u, int(x)))
            seq += 1

    propose(0)
    while len(paths) < budget and heap:
        s, _, u, x = heapq.heappop(heap)
        paths.append(paths[u] + (x,))
        score.append(-s)
        propose(len(paths) - 1)
    return set(paths)


@pytest.mark.parametrize("seed,widths,budget", [
    (0, (4, 4, 3, 2, 2), 64), (1, (4, 3, 2), 20), (2, (2, 2, 2, 2, 2, 2), 40), (3, (5,), 3),
])
def test_best_first_growth_keeps_the_same_tree(seed, widths, budget):
    """EAGLE-2-style dynamic growth and the top-M of the full expansion agree."""
    rng = np.random.default_rng(seed)
    V = 500
    rows = {}

    def row_of(tpath):
        if tpath not in rows:
            rows[tpath] = (rng.standard_normal(V) * 3).astype(np.float32)
        return rows[tpath]

    par, tok, gap, paths = _full_expansion(row_of, widths, 7)
    op, ot, src = oracle.select_topm(par[None], tok[None], gap[None], budget)
    assert {paths[int(i)] for i in src[0]} == _grow_best_first(row_of, widths, budget, 7)
    # the output is the same tree renumbered: parents map through out_src
    for j in range(1, budget):
        assert src[0, op[0, j]] == par[src[0, j]]
        assert ot[0, j] == tok[src[0, j]]


@pytest.mark.parametrize("seed", range(6))
def test_pick_is_a_subtree_above_every_dropped_node(seed):
    rng = np.random.default_rng(100 + seed)
    B, Nc = 4, 300
    par = np.stack([random_parent(rng, Nc) for _ in range(B)])
    # coarse log q so that many scores tie; some -inf; some tiny positive
    lq = -np.round(rng.exponential(1.0, (B, Nc)) * 4) / 4
    lq[rng.random((B, Nc)) < 0.05] = -np.inf
    lq[rng.random((B, Nc)) < 0.05] = 1e-17
    tok = rng.integers(0, 1000, (B, Nc))
    M = 64
    op, ot, src = oracle.select_topm(par, tok, lq, M)
    for b in range(B):
        kept = set(src[b].tolist())
        assert (np.diff(src[b]) > 0).all() and src[b, 0] == 0
        assert op[b, 0] == -1 and all(0 <= op[b, j] < j for j in range(1, M))
        assert all(int(par[b, i]) in kept for i in kept if i != 0)
        # scores along paths (products of q, compared as logs of path sums)
        score = np.zeros(Nc)
        for i in range(1, Nc):
            score[i] = score[par[b, i]] + min(lq[b, i], 0.0)
        dropped = [i for i in range(Nc) if i not in kept]
        assert min(score[list(kept)]) >= max(score[dropped])
        assert (ot[b] == tok[b, src[b]]).all()


def test_special_cases():
    Nc = 10
    chain = np.arange(-1, Nc - 1)[None]
    lq = np.log(np.linspace(0.9, 0.1, Nc))[None]
    for M in (1, 4, Nc):
        op, ot, src = oracle.select_topm(chain, np.arange(Nc)[None], lq, M)
        assert (src[0] == np.arange(M)).all() and (op[0] == np.arange(-1, M - 1)).all()
    star = np.r_[-1, np.zeros(Nc - 1, int)][None]
    lq = np.log(np.r_[1.0, 0.1, 0.3, 0.2, 0.3, 0.05, 0.01, 0.4, 0.3, 0.02])[None]
    op, ot, src = oracle.select_topm(star, np.arange(Nc)[None], lq, 4)
    assert src[0].tolist() == [0, 2, 4, 7]      # 0.4, then the two 0.3 of lower index
    op, ot, src = oracle.select_topm(star, np.arange(Nc)[None], np.zeros((1, Nc)), 5)
    assert src[0].tolist() == [0, 1, 2, 3, 4]
    rng = np.random.default_rng(3)
    par = random_parent(rng, 50)[None]
    op, ot, src = oracle.select_topm(par, np.arange(50)[None], -rng.random((1, 50)), 50)
    assert (src[0] == np.arange(50)).all() and (op[0] == par[0]).all()


def test_invalid_inputs_raise():
    par = np.array([[-1, 0, 0]])
    with pytest.raises(ValueError):
        oracle.select_topm(par, par, np.zeros((1, 3)), 0)
    with pytest.raises(ValueError):
        oracle.select_topm(par, par, np.zeros((1, 3)), 4)
    with pytest.raises(ValueError):
        oracle.select_topm(np.array([[-1, 2, 0]]), par, np.zeros((1, 3)), 2)
    with pytest.raises(ValueError):
        oracle.select_topm(par, par, np.array([[0.0, np.nan, 0.0]]), 2)


# ---- entropy-ranked widths -------------------------------------------------

def test_widths_split_the_frontier_into_equal_rank_groups():
    """With F a multiple of the number of widths, each width goes to exactly
    F / span nodes, and a node never gets fewer branches than one of lower
    entropy (the glossary's entropy-based branching)."""
    rng = np.random.default_rng(7)
    for F, (lo, hi) in [(8, (1, 4)), (40, (1, 4)), (12, (2, 3)), (30, (0, 2))]:
        h = rng.exponential(2.0, (5, F))
        w = oracle.widths_by_entropy(h, lo, hi)
        for b in range(5):
            counts = np.bincount(w[b] - lo, minlength=hi - lo + 1)
            assert (counts == F // (hi - lo + 1)).all()
            order = np.argsort(h[b], kind="stable")
            assert (np.diff(w[b][order]) >= 0).all()


def test_widths_special_cases():
    assert oracle.widths_by_entropy(np.array([[3.0]]), 1, 4).tolist() == [[1]]
    # equal entropies: rank by index
    assert oracle.widths_by_entropy(np.zeros((1, 4)), 1, 4).tolist() == [[1, 2, 3, 4]]
    assert oracle.widths_by_entropy(np.array([[5.0, 1.0, 3.0, 2.0]]), 1, 4).tolist() == [[4, 1, 3, 2]]
    # a constant width when w_min == w_max
    assert (oracle.widths_by_entropy(np.random.default_rng(1).random((2, 9)), 3, 3) == 3).all()
    # F = 5 over 4 widths: ranks 0..4 -> 1 + floor(4 r / 5) = 1, 1, 2, 3, 4
    assert sorted(oracle.widths_by_entropy(np.arange(5.0)[None], 1, 4)[0].tolist()) == [1, 1, 2, 3, 4]
    with pytest.raises(ValueError):
        oracle.widths_by_entropy(np.array([[np.nan, 1.0]]), 1, 4)
    with pytest.raises(ValueError):
        oracle.widths_by_entropy(np.zeros((1, 2)), 3, 2)
