"""Pins for the oracle's tree-topology dynamic program (CPU only).

What fixes it independently of its code:
  * brute force: over every ordered tree of up to 9 nodes (with the width and
    depth limits), the largest expected accepted count equals the program's
    value, and the program's tree has that value when scored by a separate
    path-product sum;
  * the chain: with only first children ever accepted (p = (a, 0, ...)) the
    optimum is the chain and its value is the closed form sum_{i<n} a^i, the
    pages' expected length of linear speculation less the bonus token;
  * depth 1 is the star of the min(n - 1, K) likeliest ranks;
  * more budget never lowers the value; bad arguments raise.
"""

import itertools
import math

import numpy as np
import pytest

from oracle.topology import topology, tree_value


def plane_trees(n, K, depth):
    """Every ordered rooted tree of n nodes, each node at most K children,
    depth at most `depth`, as (parent, rank) lists in breadth-first order."""
    def shapes(m, d):
        # a shape is a tuple of child shapes
        if m == 1:
            yield ()
            return
        if d == 0:
            return
        for k in range(1, min(K, m - 1) + 1):
            for sizes in compositions(m - 1, k):
                for kids in itertools.product(*[list(shapes(s, d - 1)) for s in sizes]):
                    yield tuple(kids)

    def compositions(total, parts):
        if parts == 1:
            yield (total,)
            return
        for first in range(1, total - parts + 2):
            for rest in compositions(total - first, parts - 1):
                yield (first,) + rest

    for shape in shapes(n, depth):
        parent, rank, queue = [-1], [0], [(0, shape)]
        h = 0
        while h < len(queue):
            node, sh = queue[h]
            h += 1
            for j, kid in enumerate(sh):
                parent.append(node)
                rank.append(j + 1)
                queue.append((len(parent) - 1, kid))
        yield parent, rank


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_over_all_small_trees(seed):
    rng = np.random.default_rng(seed)
    K = int(rng.integers(1, 5))
    p = np.sort(rng.uniform(0.05, 0.95, K))[::-1]
    for n in range(1, 10):
        for depth in (1, 2, 3, 8):
            trees = list(plane_trees(n, K, depth))
            if not trees:
                with pytest.raises(ValueError):
                    topology(p, n, depth)
                continue
            best = max(tree_value(pa, rk, p) for pa, rk in trees)
            parent, rank, value = topology(p, n, depth)
            assert math.isclose(value, best, rel_tol=1e-12, abs_tol=1e-15), (n, depth, value, best)
            assert math.isclose(tree_value(parent, rank, p), value, rel_tol=1e-12, abs_tol=1e-15)
            assert len(parent) == n and parent[0] == -1
            assert all(0 <= parent[i] < i for i in range(1, n))
            kids = {}
            for i in range(1, n):
                kids.setdefault(int(parent[i]), []).append(int(rank[i]))
            for ranks in kids.values():
                assert ranks == list(range(1, len(ranks) + 1)) and len(ranks) <= K


def test_unsorted_rates_are_brute_forced_too():
    p = [0.3, 0.7, 0.1]           # a later rank may be likelier: the program still finds the best
    for n in range(2, 9):
        best = max(tree_value(pa, rk, p) for pa, rk in plane_trees(n, 3, 8))
        assert math.isclose(topology(p, n, 8)[2], best, rel_tol=1e-12)


@pytest.mark.parametrize("a", [0.5, 0.8, 0.9])
@pytest.mark.parametrize("n", [2, 4, 6, 9, 40])
def test_first_children_only_give_the_chain_and_its_closed_form(a, n):
    parent, rank, value = topology([a, 0.0, 0.0, 0.0], n, n)
    assert (parent == np.arange(-1, n - 1)).all() and (rank[1:] == 1).all()
    # the pages' linear-speculation closed form (1 - a^(g+1)) / (1 - a) counts
    # the bonus token; the accepted count of n - 1 drafts is that minus 1
    closed = (1 - a ** n) / (1 - a) - 1
    assert math.isclose(value, closed, rel_tol=1e-13)


def test_depth_one_is_the_star_of_the_likeliest_ranks():
    p = [0.6, 0.3, 0.2, 0.1]
    for n in range(1, 6):
        parent, rank, value = topology(p, n, 1)
        assert (parent[1:] == 0).all()
        assert math.isclose(value, sum(p[:n - 1]), rel_tol=1e-15)


def test_more_budget_never_lowers_the_value_and_bad_arguments_raise():
    p = [0.7, 0.4, 0.2]
    vals = [topology(p, n, 6)[2] for n in range(1, 60)]
    assert all(b >= a for a, b in zip(vals, vals[1:]))
    for args in (([0.5], 0, 3), ([0.5], 4, -1), ([1.5], 4, 3), ([float("nan")], 4, 3), ([], 4, 3)):
        with pytest.raises(ValueError):
            topology(*args)
    with pytest.raises(ValueError):
        topology([0.5, 0.5], 8, 2)          # at most 1 + 2 + 4 nodes within depth 2
