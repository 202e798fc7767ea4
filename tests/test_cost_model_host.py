"""The library's host-side speedup model against the oracle's (CPU only:
these entry points run on the host and launch nothing)."""

import math

import numpy as np
import pytest

import tree_attention_verification_ancestor_amd as tav
from oracle import cost


@pytest.mark.parametrize("p", [0.0, 0.5, 0.8, 0.9, 0.97, 1.0])
@pytest.mark.parametrize("alpha,ratio", [(0.05, 0.0), (0.08, 0.0), (0.1, 0.2), (0.15, 0.05),
                                         (0.0, 0.0)])
def test_best_chain_length_matches_oracle(p, alpha, ratio):
    n, s = tav.best_chain_length(p, ratio, alpha, 200)
    rn, rs = cost.best_chain_length(p, ratio, alpha, 200)
    assert n == rn
    assert s == pytest.approx(rs, rel=1e-13)


def test_model_speedup_matches_oracle():
    rng = np.random.default_rng(2)
    for _ in range(200):
        e, r, a, n = rng.uniform(1, 10), rng.uniform(0, 1), rng.uniform(0, 0.2), int(rng.integers(0, 300))
        assert tav.model_speedup(e, r, a, n) == pytest.approx(cost.speedup(e, r, a, n), rel=1e-15)


def test_fit_alpha_matches_oracle():
    rng = np.random.default_rng(3)
    n = [1, 2, 4, 8, 16, 32, 64]
    t = 60.0 * (1 + 0.04 * (np.array(n) - 1)) * rng.uniform(0.97, 1.03, len(n))
    assert tav.fit_alpha(n, t) == pytest.approx(cost.alpha_from_times(n, t), rel=1e-12)


def test_bad_input():
    assert math.isnan(tav.model_speedup(1.0, -0.1, 0.1, 4))
    assert math.isnan(tav.model_speedup(1.0, 0.0, 0.1, -1))
    assert tav.best_chain_length(1.2, 0.0, 0.1, 10)[0] == 0
    assert tav.best_chain_length(0.8, 0.0, 0.1, 0)[0] == 0
    assert tav.best_chain_length(0.8, 0.0, float("inf"), 10)[0] == 0
    assert math.isnan(tav.fit_alpha([2, 4], [1.0, 2.0]))
    assert math.isnan(tav.fit_alpha([1], [1.0]))
    assert math.isnan(tav.fit_alpha([1, 2], [1.0, -2.0]))


def test_verify_speedup_matches_the_oracle_and_rejects_bad_input():
    import math
    from oracle.cost import verify_speedup
    cases = [(3.0, 0.0, 32, 218e6, 525e6, 1, 16, 26.5, 36.6, 20.0, 30.0, 8000.0, 2500.0),
             (2.6, 0.1, 32, 218e6, 525e6, 128, 6, 341.0, 326.0, 300.0, 200.0, 6200.0, 2500.0),
             (4.4, 0.0, 80, 855e6, 1050e6, 8, 64, 153.0, 50.0, 100.0, 20.0, 8000.0, 2500.0)]
    for c in cases:
        got = tav.verify_speedup(*c)
        want = verify_speedup(*c)
        for g, w in zip(got, want):
            assert math.isclose(g, w, rel_tol=1e-12), (c, got, want)
    bad = list(cases[0])
    for i, v in ((0, -1.0), (2, 0), (5, 0), (6, 0), (7, float("nan")), (11, 0.0)):
        b = list(bad)
        b[i] = v
        assert math.isnan(tav.verify_speedup(*b)[0]), i
