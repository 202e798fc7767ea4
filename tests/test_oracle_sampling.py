"""Pins for the oracle's Philox uniforms and rejection-sampling walk (CPU only).

Independent routes to the same facts:
  * Philox words: numpy.random.Philox (a separate Philox4x64-10 implementation);
  * single-node steps: scipy softmax + numpy cumsum/searchsorted;
  * acceptance direction and uniform mapping: one-hot drafts, where the walk
    must accept exactly when the node's uniform is below p(x);
  * losslessness (radar-34b blog section 2; LLM Primer ch. 9 section 9.1):
    a chi-square test over 10^6 trials that the first emitted token follows p;
  * the linear-speculation closed form (jisaku.com glossary, linear vs tree
    table): mean emitted tokens of a gamma-draft chain with constant
    acceptance alpha is (1 - alpha^(gamma+1)) / (1 - alpha).
"""

import numpy as np
import pytest
import scipy.special

import oracle

# chi-square critical values at p = 0.001 by degrees of freedom
CHI2_DOF_P001 = {3: 16.27, 5: 20.52, 7: 24.32}
CHI2_7DOF_P001 = CHI2_DOF_P001[7]


def _numpy_block(ctr, key):
    """Philox4x64-10 block at counter ``ctr`` via numpy (which steps the
    counter once before its first block, so start one below)."""
    c = sum(int(w) << (64 * k) for k, w in enumerate(ctr))
    c = (c - 1) % (1 << 256)
    start = [(c >> (64 * k)) & ((1 << 64) - 1) for k in range(4)]
    return np.random.Philox(counter=np.array(start, dtype=np.uint64),
                            key=np.array([int(key[0]), int(key[1])], dtype=np.uint64)).random_raw(4)


def _u(w):
    return float(int(w) >> 40) / 16777216.0


@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 1, 2, 0), (7, 0)),
    ((2**64 - 1, 3, 9, 0), (123456789, 0)),
    ((0, 0, 0, 1), (2**63 + 5, 2**40)),
    ((17, 2**63, 2**64 - 1, 2**64 - 1), (1, 1)),
])
def test_philox_matches_numpy(ctr, key):
    ours = oracle.philox4x64_10(np.array([ctr], np.uint64), key)[0]
    np.testing.assert_array_equal(ours, _numpy_block(ctr, key))


def test_node_uniforms_follow_counter_convention():
    seed, offset, B, N = 42, 9, 3, 7
    u = oracle.node_uniforms(seed, offset, B, N)
    for b in range(B):
        for i in range(N):
            w = _numpy_block((offset, b, i, 0), (seed, 0))
            assert u[b, i, 0] == _u(w[0]) and u[b, i, 1] == _u(w[1])
    assert ((u >= 0) & (u < 1)).all()


def _leaf_only(B, V, rng, sigma=2.0):
    tl = (rng.standard_normal((B, 1, V)) * sigma).astype(np.float32)
    dl = (rng.standard_normal((B, 1, V)) * sigma).astype(np.float32)
    parent = np.full((B, 1), -1, np.int32)
    token = np.zeros((B, 1), np.int32)
    return tl, dl, parent, token


@pytest.mark.parametrize("T", [1.0, 0.7, 1.9])
def test_single_node_is_inverse_cdf(T):
    """N = 1: the step reduces to one inverse-CDF draw from softmax(l / T)."""
    rng = np.random.default_rng(0)
    B, V = 2000, 1000
    tl, dl, parent, token = _leaf_only(B, V, rng)
    res = oracle.verify_walk(tl, dl, parent, token, T, seed=3, offset=11)
    p = scipy.special.softmax(tl[:, 0].astype(np.float64) / T, axis=-1)
    c = np.cumsum(p, axis=-1)
    mismatched = 0
    for b in range(B):
        r = _u(_numpy_block((11, b, 0, 0), (3, 0))[1])
        k = int(np.searchsorted(c[b], r * c[b, -1], side="right"))
        if res.out_tokens[b, 0] != k:
            assert res.near[b] > 0          # only a draw at a boundary may differ
            mismatched += 1
    assert mismatched <= 1e-4 * res.draws.sum()
    assert (res.n_accepted == 0).all()
    assert (res.path[:, 0] == 0).all()


def test_zero_probability_tokens_never_drawn():
    rng = np.random.default_rng(1)
    B, V = 3000, 64
    tl, dl, parent, token = _leaf_only(B, V, rng)
    tl[:, :, ::2] = -np.inf          # even tokens have p = 0
    tl[:, :, 0] = -np.inf
    res = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=0)
    assert (res.out_tokens[:, 0] % 2 == 1).all()


def test_identical_draft_accepts_first_children_to_a_leaf():
    rng = np.random.default_rng(2)
    from synth import random_parent
    B, N, V = 60, 30, 50
    parent = np.stack([random_parent(rng, N) for _ in range(B)])
    tl = (rng.standard_normal((B, N, V)) * 2).astype(np.float32)
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    res = oracle.verify_walk(tl, tl.copy(), parent, token, 1.0, seed=5)
    for b in range(B):
        u, path = 0, [0]
        while True:
            kids = [c for c in range(N) if parent[b, c] == u]
            if not kids:
                break
            u = min(kids)
            path.append(u)
        m = len(path) - 1
        assert res.n_accepted[b] == m
        assert list(res.path[b, :m + 1]) == path and (res.path[b, m + 1:] == -1).all()
        assert list(res.out_tokens[b, :m]) == [int(token[b, c]) for c in path[1:]]


def test_zero_target_probability_always_rejected():
    rng = np.random.default_rng(3)
    B, V = 500, 40
    parent = np.tile(np.array([-1, 0, 0, 0], np.int32), (B, 1))
    token = np.tile(np.array([0, 3, 7, 11], np.int32), (B, 1))
    tl = (rng.standard_normal((B, 4, V))).astype(np.float32)
    dl = (rng.standard_normal((B, 4, V))).astype(np.float32)
    tl[:, 0, [3, 7, 11]] = -np.inf
    res = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=9)
    assert (res.n_accepted == 0).all()
    assert not np.isin(res.out_tokens[:, 0], [3, 7, 11]).any()


@pytest.mark.parametrize("alpha", [0.1, 0.5, 0.93])
def test_one_hot_draft_accepts_iff_uniform_below_p(alpha):
    """q is one-hot on x and p(x) = alpha: accept exactly when u_acc < alpha."""
    B, V, x = 20000, 16, 5
    t = np.full(V, np.log((1 - alpha) / (V - 1)))
    t[x] = np.log(alpha)
    tl = np.tile(t.astype(np.float32), (B, 2, 1))
    d = np.full(V, -np.inf, np.float32)
    d[x] = 0.0
    dl = np.tile(d, (B, 2, 1))
    parent = np.tile(np.array([-1, 0], np.int32), (B, 1))
    token = np.tile(np.array([0, x], np.int32), (B, 1))
    res = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=77, offset=1)
    u_acc = np.array([_u(_numpy_block((1, b, 1, 0), (77, 0))[0]) for b in range(B)])
    px = scipy.special.softmax(t)[x]
    decided = np.abs(u_acc - px) > 1e-6
    assert ((res.n_accepted == 1) == (u_acc < px))[decided].all()
    assert abs((res.n_accepted == 1).mean() - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / B)


def _chi2(counts, probs):
    n = counts.sum()
    exp = probs * n
    return float(((counts - exp) ** 2 / exp).sum())


def _lossless_trial(p_logits, q_logits, k, T, trials, seed):
    """Root with k leaf children drafted i.i.d. from q; returns first-token counts."""
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
    token[:, 1:] = rng.choice(V, size=(trials, k), p=q)
    res = oracle.verify_walk(tl, dl, parent, token, T, seed=seed, offset=0)
    first = res.out_tokens[:, 0]
    return np.bincount(first, minlength=V), res


CASES = {
    "random": lambda r: (r.standard_normal(8) * 1.5, r.standard_normal(8) * 1.5),
    "disjoint": lambda r: (np.r_[r.standard_normal(4), [-np.inf] * 4],
                           np.r_[[-np.inf] * 4, r.standard_normal(4)]),
    "q_zero_where_p_positive": lambda r: (r.standard_normal(8), np.r_[r.standard_normal(6), [-np.inf] * 2]),
}


@pytest.mark.parametrize("case,k,T", [
    ("random", 1, 1.0), ("random", 2, 1.0), ("random", 3, 1.0), ("random", 3, 0.7),
    ("disjoint", 2, 1.0), ("q_zero_where_p_positive", 3, 1.0),
])
def test_chi_square_output_distribution_is_p(case, k, T):
    rng = np.random.default_rng(100 + k)
    pl, ql = (a.astype(np.float32) for a in CASES[case](rng))
    counts, res = _lossless_trial(pl, ql, k, T, 10**6, seed=k)
    p = scipy.special.softmax(pl.astype(np.float64) / T)
    live = p > 0
    assert counts[~live].sum() == 0
    stat = _chi2(counts[live], p[live])
    assert stat < CHI2_DOF_P001[int(live.sum()) - 1], stat


def test_chi_square_detects_a_lossy_rule():
    """Sanity of the statistic: sampling straight from q fails it."""
    rng = np.random.default_rng(7)
    pl, ql = (a.astype(np.float32) for a in CASES["random"](rng))
    q = scipy.special.softmax(ql.astype(np.float64))
    p = scipy.special.softmax(pl.astype(np.float64))
    counts = np.bincount(rng.choice(8, size=10**6, p=q), minlength=8)
    assert _chi2(counts, p) > CHI2_7DOF_P001


@pytest.mark.parametrize("gamma,alpha,trials", [
    (1, 0.5, 200000), (3, 0.8, 200000), (5, 0.8, 10**6), (8, 0.9, 200000), (5, 0.5, 200000),
    (8, 0.8, 200000),
])
def test_linear_closed_form_expected_length(gamma, alpha, trials):
    """Chain of gamma drafts with constant acceptance alpha.

    q is uniform on tokens 0..3; p = alpha * q + (1 - alpha) * uniform(4..7),
    so min(1, p/q) = alpha for every draft. Mean emitted tokens (accepted + 1)
    must sit within 5 standard errors of (1 - alpha^(gamma+1)) / (1 - alpha).
    """
    rng = np.random.default_rng(gamma * 10 + int(alpha * 10))
    V, N = 8, gamma + 1
    pl = np.log(np.r_[[alpha / 4] * 4, [(1 - alpha) / 4] * 4]).astype(np.float32)
    ql = np.r_[[0.0] * 4, [-np.inf] * 4].astype(np.float32)
    tl = np.empty((trials, N, V), np.float32)
    tl[:] = pl
    dl = np.empty((trials, N, V), np.float32)
    dl[:] = ql
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (trials, 1))
    token = rng.integers(0, 4, (trials, N)).astype(np.int32)
    res = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=gamma, offset=3)
    emitted = res.n_accepted.astype(np.float64) + 1
    expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    se = emitted.std() / np.sqrt(trials)
    assert abs(emitted.mean() - expect) < 5 * se, (emitted.mean(), expect, se)
    if gamma == 5 and alpha == 0.8:
        assert abs(expect - 3.68928) < 1e-5


def test_invalid_inputs_rejected():
    tl = np.zeros((1, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.verify_walk(tl, tl, np.array([[-1, 2, 0]], np.int32), np.zeros((1, 3), np.int32))
    with pytest.raises(ValueError):
        oracle.verify_walk(tl, tl, np.array([[-1, 0, 0]], np.int32), np.array([[0, 4, 0]], np.int32))
    bad = tl.copy()
    bad[0, 0, :] = -np.inf
    with pytest.raises(ValueError):
        oracle.verify_walk(bad, tl, np.array([[-1, 0, 0]], np.int32), np.zeros((1, 3), np.int32))
    bad[0, 0, :] = np.nan
    with pytest.raises(ValueError):
        oracle.verify_walk(bad, tl, np.array([[-1, 0, 0]], np.int32), np.zeros((1, 3), np.int32))


def _zero_uniform_counters():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "zero_uniforms.txt")
    found = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            kind, seed, offset, node = line.split()
            found[kind] = (int(seed), int(offset), int(node))
    return found


def test_zero_uniform_counters_are_zero_under_numpy():
    z = _zero_uniform_counters()
    seed, off, node = z["acceptance"]
    assert int(_numpy_block((off, 0, node, 0), (seed, 0))[0]) >> 40 == 0
    seed, off, node = z["resample"]
    assert int(_numpy_block((off, 0, node, 0), (seed, 0))[1]) >> 40 == 0


def test_resample_at_zero_uniform_skips_zero_mass_tokens():
    """Strict C(k) > r*Z: with r = 0 the draw is the first token with mass."""
    seed, off, _ = _zero_uniform_counters()["resample"]
    tl = np.array([[[-np.inf, -np.inf, 0.3, 1.0, -np.inf, 2.0, 0.0, 0.1]]], np.float32)
    res = oracle.verify_walk(tl, tl, np.array([[-1]], np.int32), np.zeros((1, 1), np.int32),
                             1.0, seed=seed, offset=off)
    assert res.out_tokens[0, 0] == 2


def test_accept_at_zero_uniform_still_rejects_zero_mass_draft():
    """Strict r*q(x) < p(x): with r = 0 a draft with p(x) = 0 is still rejected,
    and a draft with p(x) > 0 is accepted."""
    seed, off, node = _zero_uniform_counters()["acceptance"]
    assert node == 1
    V = 8
    dl = np.zeros((1, 2, V), np.float32)
    tl = np.zeros((1, 2, V), np.float32)
    tl[0, 0, 4] = -np.inf
    parent = np.array([[-1, 0]], np.int32)
    res = oracle.verify_walk(tl, dl, parent, np.array([[0, 4]], np.int32), 1.0, seed=seed, offset=off)
    assert res.n_accepted[0] == 0 and res.out_tokens[0, 0] != 4
    res = oracle.verify_walk(tl, dl, parent, np.array([[0, 5]], np.int32), 1.0, seed=seed, offset=off)
    assert res.n_accepted[0] == 1 and res.out_tokens[0, 0] == 5
