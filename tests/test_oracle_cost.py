"""Pins for the oracle's speedup model (CPU only).

  * the pages' worked numbers (tests/golden/speedup_model.txt, LLM Primer
    ch. 9 section 9.3): the best chain length at acceptance 0.8 and 0.9, and
    the 1/alpha ceiling as acceptance approaches 1;
  * the linear-speculation closed form (jisaku.com glossary) for the
    expected emitted tokens of a chain;
  * special cases of the tree estimate: a chain with constant q reduces to
    the chain formula, a star to 1 + the sum of its q;
  * the overhead fit recovers alpha exactly from times that follow the model.
"""

import math
import os

import numpy as np
import pytest

from oracle import cost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "speedup_model.txt")


def _golden():
    optima, limits = [], []
    for line in open(GOLDEN):
        f = line.split("#")[0].split()
        if len(f) == 5:
            optima.append((float(f[0]), float(f[1]), float(f[2]), int(f[3]), int(f[4])))
        elif len(f) == 2:
            limits.append((float(f[0]), float(f[1])))
    return optima, limits


def test_best_chain_length_matches_the_pages():
    optima, _ = _golden()
    assert len(optima) == 2
    for p, alpha, ratio, lo, hi in optima:
        n, s = cost.best_chain_length(p, ratio, alpha, 64)
        assert lo <= n <= hi, (p, n)
        # a longer chain past the optimum is slower: the alpha*N term wins
        assert cost.speedup(cost.chain_expected_emitted(p, 40), ratio, alpha, 40) < s


def test_speedup_ceiling_is_one_over_alpha():
    _, limits = _golden()
    assert len(limits) == 2
    for alpha, limit in limits:
        assert limit == pytest.approx(1.0 / alpha)
        # p = 1 accepts everything: (N + 1) / (1 + alpha N) rises to 1/alpha
        prev = 0.0
        for n in (1, 10, 100, 10**4, 10**6):
            s = cost.speedup(n + 1, 0.0, alpha, n)
            assert prev < s < limit
            prev = s
        assert prev == pytest.approx(limit, rel=1e-4)
        # and the best chain at p near 1 approaches it from below
        n, s = cost.best_chain_length(0.999, 0.0, alpha, 4000)
        assert 0.8 * limit < s < limit


@pytest.mark.parametrize("p", [0.0, 0.3, 0.8, 0.95])
def test_chain_expected_emitted_closed_form(p):
    for n in (0, 1, 5, 30):
        closed = (1 - p ** (n + 1)) / (1 - p)
        assert cost.chain_expected_emitted(p, n) == pytest.approx(closed, rel=1e-13)


def test_tree_estimate_special_cases():
    n = 9
    chain = np.arange(-1, n - 1)
    p = 0.7
    lq = np.full(n, math.log(p))
    assert cost.tree_expected_emitted(chain, lq) == pytest.approx(
        cost.chain_expected_emitted(p, n - 1), rel=1e-13)
    star = np.r_[-1, np.zeros(5, int)]
    q = np.array([1.0, 0.1, 0.2, 0.3, 0.05, 0.25])
    assert cost.tree_expected_emitted(star, np.log(q)) == pytest.approx(1 + q[1:].sum(), rel=1e-13)
    assert cost.tree_expected_emitted(np.array([-1]), np.array([0.0])) == 1.0


def test_alpha_fit_recovers_the_model():
    n = np.array([1, 2, 4, 8, 16, 32, 64])
    for alpha in (0.02, 0.1):
        t = 57.0 * (1 + alpha * (n - 1))
        assert cost.alpha_from_times(n, t) == pytest.approx(alpha, rel=1e-12)
    with pytest.raises(ValueError):
        cost.alpha_from_times([2, 4], [1.0, 2.0])


def test_speedup_falls_with_overheads():
    e = cost.chain_expected_emitted(0.8, 6)
    assert cost.speedup(e, 0.0, 0.1, 6) > cost.speedup(e, 0.2, 0.1, 6) > cost.speedup(e, 0.2, 0.15, 6)


# --- the batch-aware model (a whole decode step as alpha's baseline) -------

def _vs(E=3.0, B=1, n=16, av=0.0, sv=0.0, ad=0.0, sd=0.0, draft=0.0):
    from oracle.cost import verify_speedup
    return verify_speedup(E, draft, 32, 218e6, 525e6, B, n, av, sv, ad, sd, 8000.0, 2500.0)


def test_verify_model_is_the_plain_model_when_verification_costs_a_decode_step():
    # n = 1 with the decode step's own times: T_verify = T_decode, alpha = 0
    s, alpha, td, tv = _vs(E=1.7, n=1, av=20.0, sv=30.0, ad=20.0, sd=30.0)
    assert alpha == 0.0 and td == tv and s == 1.7


def test_weight_bound_batch_has_no_overhead_from_the_linear_layers():
    # B n tokens still read the weights in less time than their FLOPs take
    # (2 params B n / MFMA < 2 params / HBM while B n < 312): alpha = 0
    s, alpha, td, tv = _vs(E=2.5, B=4, n=16)
    assert alpha == 0.0 and s == 2.5


def test_compute_bound_batch_costs_n_decode_steps():
    # at B = 4096 both passes are MFMA-bound: T_verify / T_decode = n exactly
    s, alpha, td, tv = _vs(E=2.0, B=4096, n=8)
    assert abs(tv / td - 8.0) < 1e-12
    assert abs(s - 2.0 / 8.0) < 1e-12


def test_speedup_falls_as_the_batch_grows():
    prev = None
    for B in (1, 4, 16, 64, 128, 256, 1024):
        s = _vs(E=3.0, B=B, n=16, av=30.0 + B, sv=40.0 + B, ad=20.0 + B / 4, sd=30.0 + B / 4)[0]
        if prev is not None:
            assert s <= prev + 1e-12
        prev = s
