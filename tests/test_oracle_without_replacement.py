"""Pins for the oracle's without-replacement sibling rule (CPU only).

Under this rule the children of a node are drawn from q_u without
replacement, and after a child with token x is rejected, x leaves q (its
entry set to zero, the rest renormalised) before the next sibling is tried;
the rejection step itself is the radar-34b blog's (section 2): accept with
min(1, p/q), else continue from the normalised positive part of p - q.

What fixes the rule independently of its code:
  * losslessness, the property the pages' rejection step exists to keep
    (radar-34b blog section 2; LLM Primer ch. 9 section 9.1): over 10^6
    seeded trials with siblings drawn without replacement (Gumbel top-k, the
    sequential without-replacement order), the first emitted token follows p
    by a chi-square test;
  * the same test rejects the i.i.d. rule on those drafts, and the
    without-replacement rule on i.i.d. drafts, so the q update is neither a
    no-op nor harmless where it does not belong;
  * chains (one child per node) never meet a second sibling, so both rules
    give identical walks;
  * two tokens both drafted: one of them is always accepted.
"""

import numpy as np
import pytest
import scipy.special

import oracle

CHI2_DOF_P001 = {3: 16.27, 5: 20.52, 7: 24.32}


def _chi2(counts, probs):
    n = counts.sum()
    exp = probs * n
    return float(((counts - exp) ** 2 / exp).sum())


def _draft_without_replacement(rng, q, trials, k):
    """k distinct tokens per trial in sequential without-replacement order:
    the k largest of log q + Gumbel noise, largest first."""
    with np.errstate(divide="ignore"):
        logq = np.log(q)
    keys = logq[None, :] + rng.gumbel(size=(trials, q.shape[0]))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def _trial(p_logits, q_logits, k, T, trials, seed, draft_wor, rule_wor):
    rng = np.random.default_rng(seed)
    V = p_logits.shape[0]
    N = k + 1
    q = scipy.special.softmax(q_logits.astype(np.float64) / T)
    tl = np.empty((trials, N, V), np.float32)
    tl[:] = p_logits
    dl = np.empty((trials, N, V), np.float32)
    dl[:] = q_logits
    parent = np.tile(np.array([-1] + [0] * k, np.int32), (trials, 1))
    token = np.zeros((trials, N), np.int32)
    if draft_wor:
        token[:, 1:] = _draft_without_replacement(rng, q, trials, k)
    else:
        token[:, 1:] = rng.choice(V, size=(trials, k), p=q)
    res = oracle.verify_walk(tl, dl, parent, token, T, seed=seed, offset=0,
                             without_replacement=rule_wor)
    return np.bincount(res.out_tokens[:, 0], minlength=V), res


CASES = {
    "random": lambda r: (r.standard_normal(8) * 1.5, r.standard_normal(8) * 1.5),
    "peaked_draft": lambda r: (r.standard_normal(8), np.r_[[3.0], r.standard_normal(7)]),
    "disjoint": lambda r: (np.r_[r.standard_normal(4), [-np.inf] * 4],
                           np.r_[[-np.inf] * 4, r.standard_normal(4)]),
    "q_zero_where_p_positive": lambda r: (r.standard_normal(8),
                                          np.r_[r.standard_normal(6), [-np.inf] * 2]),
}


@pytest.mark.parametrize("case,k,T", [
    ("random", 2, 1.0), ("random", 3, 1.0), ("random", 4, 0.7), ("peaked_draft", 3, 1.0),
    ("disjoint", 3, 1.0), ("q_zero_where_p_positive", 4, 1.0),
])
def test_chi_square_output_distribution_is_p(case, k, T):
    rng = np.random.default_rng(200 + k)
    pl, ql = (a.astype(np.float32) for a in CASES[case](rng))
    counts, _ = _trial(pl, ql, k, T, 10**6, seed=30 + k, draft_wor=True, rule_wor=True)
    p = scipy.special.softmax(pl.astype(np.float64) / T)
    live = p > 0
    assert counts[~live].sum() == 0
    stat = _chi2(counts[live], p[live])
    assert stat < CHI2_DOF_P001[int(live.sum()) - 1], stat


@pytest.mark.parametrize("draft_wor,rule_wor", [(True, False), (False, True)])
def test_mismatched_rule_is_detected(draft_wor, rule_wor):
    """A walk whose sibling rule does not match how siblings were drawn is
    lossy, and the statistic sees it."""
    rng = np.random.default_rng(9)
    pl, ql = (a.astype(np.float32) for a in CASES["peaked_draft"](rng))
    counts, _ = _trial(pl, ql, 3, 1.0, 10**6, seed=4, draft_wor=draft_wor, rule_wor=rule_wor)
    p = scipy.special.softmax(pl.astype(np.float64))
    assert _chi2(counts, p) > 10 * CHI2_DOF_P001[7]


def test_chains_identical_under_both_rules():
    rng = np.random.default_rng(5)
    B, N, V = 64, 7, 50
    tl = (rng.standard_normal((B, N, V)) * 2).astype(np.float32)
    dl = (tl + rng.standard_normal((B, N, V))).astype(np.float32)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    a = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=2, offset=3)
    b = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=2, offset=3,
                           without_replacement=True)
    assert (a.path == b.path).all() and (a.out_tokens == b.out_tokens).all()
    assert (a.n_accepted == b.n_accepted).all()


def test_both_tokens_drafted_always_accepts_one():
    """V = 2 with both tokens as children: after the first is rejected the
    draft is the other token with certainty and the residual is that token
    alone, so the second child is accepted every time."""
    rng = np.random.default_rng(11)
    B, V = 4000, 2
    tl = np.zeros((B, 3, V), np.float32)
    dl = np.zeros((B, 3, V), np.float32)
    tl[:, 0] = rng.standard_normal((B, V)) * 2
    dl[:, 0] = rng.standard_normal((B, V)) * 2
    parent = np.tile(np.array([-1, 0, 0], np.int32), (B, 1))
    token = np.zeros((B, 3), np.int32)
    token[:, 1] = rng.integers(0, 2, B)
    token[:, 2] = 1 - token[:, 1]
    res = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=8, offset=0,
                             without_replacement=True)
    assert (res.n_accepted == 1).all()
    assert (res.out_tokens[:, 0] == token[np.arange(B), res.path[:, 1]]).all()
