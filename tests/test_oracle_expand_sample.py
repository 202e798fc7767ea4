"""Pins for the oracle's sampled expansion (CPU only).

What fixes it independently of its code:
  * one draw (k = 1) is a draw from q: first-token frequencies over 2*10^5
    rows (each row its own Philox counters) pass a chi-square test;
  * two draws are sequential draws without replacement: ordered pairs (a, b)
    appear with probability q_a q_b / (1 - q_a) (chi-square over all pairs);
  * the tree it builds is one for which the without-replacement walk is
    lossless: a root with k sampled children, walked by the oracle's
    without-replacement rule, emits first tokens that follow p, and the
    i.i.d. rule on the same children fails the same test;
  * log q and the entropy are expand_topk's for the chosen tokens, and the
    draws depend only on (seed, offset, row, token);
  * the uniforms: SplitMix64 gives the published outputs for seed 0
    (tests/golden/splitmix64_seed0.txt); the Gumbel noise built from the
    uniforms follows the standard Gumbel law (Kolmogorov-Smirnov over 10^6
    tokens); the high words of the two tokens sharing a SplitMix output, and
    the low bits of the tokens sharing a Philox word, are uncorrelated; the
    keys are x/T + G in float64.
"""
import os

import numpy as np
import pytest
import scipy.special

import oracle

CHI2_P001 = {4: 18.47, 5: 20.52, 7: 24.32, 19: 43.82}


def _chi2(counts, probs):
    n = counts.sum()
    exp = probs * n
    return float(((counts - exp) ** 2 / exp).sum())


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_one_draw_follows_q(T):
    rng = np.random.default_rng(1)
    V, R = 8, 200000
    row = (rng.standard_normal(V) * 1.2).astype(np.float32)
    tok, _, _ = oracle.expand_sample(np.tile(row, (R, 1)), 1, T, seed=3, offset=0)
    q = scipy.special.softmax(row.astype(np.float64) / T)
    assert _chi2(np.bincount(tok[:, 0], minlength=V), q) < CHI2_P001[V - 1]


def test_two_draws_are_without_replacement():
    rng = np.random.default_rng(2)
    V, R = 5, 200000
    row = (rng.standard_normal(V) * 1.0).astype(np.float32)
    tok, _, _ = oracle.expand_sample(np.tile(row, (R, 1)), 2, 1.0, seed=9, offset=4)
    assert (tok[:, 0] != tok[:, 1]).all()
    q = scipy.special.softmax(row.astype(np.float64))
    cells = [(a, b) for a in range(V) for b in range(V) if a != b]
    probs = np.array([q[a] * q[b] / (1 - q[a]) for a, b in cells])
    index = {c: i for i, c in enumerate(cells)}
    counts = np.zeros(len(cells))
    for a, b in zip(tok[:, 0], tok[:, 1]):
        counts[index[(int(a), int(b))]] += 1
    assert _chi2(counts, probs) < CHI2_P001[19]


@pytest.mark.parametrize("k", [2, 3])
def test_sampled_children_make_the_without_replacement_walk_lossless(k):
    rng = np.random.default_rng(10 + k)
    V, R = 6, 200000
    pl = (rng.standard_normal(V) * 1.2).astype(np.float32)
    ql = np.r_[[2.5], rng.standard_normal(V - 1)].astype(np.float32)
    tok, _, _ = oracle.expand_sample(np.tile(ql, (R, 1)), k, 1.0, seed=5, offset=1)
    tl = np.broadcast_to(pl, (R, k + 1, V)).copy()
    dl = np.broadcast_to(ql, (R, k + 1, V)).copy()
    parent = np.tile(np.array([-1] + [0] * k, np.int32), (R, 1))
    token = np.zeros((R, k + 1), np.int32)
    token[:, 1:] = tok
    p = scipy.special.softmax(pl.astype(np.float64))
    wor = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=6, offset=0,
                             without_replacement=True)
    assert _chi2(np.bincount(wor.out_tokens[:, 0], minlength=V), p) < CHI2_P001[V - 1]
    iid = oracle.verify_walk(tl, dl, parent, token, 1.0, seed=6, offset=0)
    assert _chi2(np.bincount(iid.out_tokens[:, 0], minlength=V), p) > 10 * CHI2_P001[V - 1]


def test_logq_entropy_and_determinism():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((20, 300)) * 3).astype(np.float32)
    x[3, :100] = -np.inf
    tok, lq, ent = oracle.expand_sample(x, 5, 0.8, seed=1, offset=2)
    q = oracle.softmax(x, 0.8)
    for r in range(20):
        assert len(set(tok[r].tolist())) == 5
        np.testing.assert_allclose(lq[r], np.log(q[r, tok[r]]), rtol=0, atol=1e-12)
    _, _, ent_top = oracle.expand_topk(x, 5, 0.8)
    np.testing.assert_allclose(ent, ent_top, rtol=0, atol=1e-12)
    again, _, _ = oracle.expand_sample(x, 5, 0.8, seed=1, offset=2)
    np.testing.assert_array_equal(tok, again)
    other, _, _ = oracle.expand_sample(x, 5, 0.8, seed=1, offset=3)
    assert (other != tok).any(axis=1).mean() > 0.5
    # a row's draws depend on its own counters only
    sub, _, _ = oracle.expand_sample(x[:4], 5, 0.8, seed=1, offset=2)
    np.testing.assert_array_equal(sub, tok[:4])
    with pytest.raises(ValueError):
        bad = x.copy()
        bad[2, 7] = np.nan
        oracle.expand_sample(bad, 2, 1.0, 0, 0)


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.txt")


def test_splitmix64_published_outputs():
    from oracle.expand import SPLITMIX_GAMMA, splitmix64
    want = [int(line.split()[1], 16) for line in open(GOLDEN)
            if line.strip() and not line.startswith("#")]
    states = np.array([(SPLITMIX_GAMMA * (i + 1)) % 2**64 for i in range(len(want))], np.uint64)
    assert [int(z) for z in splitmix64(states)] == want


def test_gumbel_noise_follows_the_gumbel_law():
    import scipy.stats
    from oracle.expand import gumbel_uniforms
    u = gumbel_uniforms(8, 125000, seed=7, offset=3).ravel()
    assert (u > 0).all() and (u < 1).all()
    g = -np.log(-np.log(u))
    assert scipy.stats.kstest(g, scipy.stats.gumbel_r.cdf).pvalue > 1e-3
    # on the 53-bit grid: (u 2^53 - 1/2) is an integer
    m = u * 2.0 ** 53 - 0.5
    assert (m[u < 0.5] == np.floor(m[u < 0.5])).all()


def test_uniform_words_are_not_shared_or_correlated():
    from oracle.expand import gumbel_uniforms
    u = gumbel_uniforms(4, 1 << 16, seed=1, offset=0)
    # tokens 2i and 2i+1 share a SplitMix output; 8j..8j+7 share a Philox block
    for a, b in ((0, 1), (0, 4), (1, 5), (3, 7), (0, 8)):
        x, y = u[:, a::16].ravel(), u[:, b::16].ravel()
        assert abs(np.corrcoef(x, y)[0, 1]) < 0.02, (a, b)
        assert (x != y).all()
    # rows and offsets give different streams
    assert (gumbel_uniforms(2, 64, 1, 0)[0] != gumbel_uniforms(2, 64, 1, 0)[1]).all()
    assert (gumbel_uniforms(1, 64, 1, 0) != gumbel_uniforms(1, 64, 1, 1)).all()


def test_keys_are_x_over_T_plus_gumbel_in_float64():
    from oracle.expand import gumbel_uniforms
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((3, 500)) * 2).astype(np.float32)
    k = oracle.gumbel_keys(x, 0.7, 5, 6)
    assert k.dtype == np.float64
    u = gumbel_uniforms(3, 500, 5, 6)
    np.testing.assert_array_equal(k, x.astype(np.float64) / 0.7 - np.log(-np.log(u)))
