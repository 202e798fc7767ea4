"""Pins of the oracle's tree expansion (top-k draft tokens, log q, entropy).

Checked against what mathematics fixes: a uniform row has entropy log V and
every log q = -log V; a one-hot row (one finite logit) has entropy 0 and log
q = 0 at its token; the top-k of a row are its k largest logits with ties to
the lower token (brute force by sorting pairs); entropy is invariant to
permuting the row and to adding a constant; temperature T equals scaling the
logits by 1/T; -inf logits contribute nothing.
"""

import math

import numpy as np
import pytest

import oracle


def test_uniform_row():
    V = 1000
    tok, logq, ent = oracle.expand_topk(np.zeros((1, V), np.float32), 5)
    np.testing.assert_array_equal(tok[0], [0, 1, 2, 3, 4])
    np.testing.assert_allclose(logq[0], -math.log(V), rtol=0, atol=1e-12)
    assert abs(ent[0] - math.log(V)) < 1e-12


def test_one_hot_row():
    row = np.full((1, 50), -np.inf, np.float32)
    row[0, 17] = 3.0
    tok, logq, ent = oracle.expand_topk(row, 1)
    assert tok[0, 0] == 17 and logq[0, 0] == 0.0 and ent[0] == 0.0


@pytest.mark.parametrize("seed", range(4))
def test_topk_is_largest_logits_ties_to_lower_token(seed):
    rng = np.random.default_rng(seed)
    R, V, k = 6, 300, 8
    x = np.round(rng.standard_normal((R, V)) * 2, 1).astype(np.float32)   # many ties
    tok, logq, _ = oracle.expand_topk(x, k)
    for r in range(R):
        pairs = sorted(((-float(x[r, i]), i) for i in range(V)))[:k]
        assert [i for _, i in pairs] == tok[r].tolist()
        assert (np.diff(logq[r]) <= 0).all()


@pytest.mark.parametrize("T", [1.0, 0.5, 2.0])
def test_entropy_invariances_and_temperature(T):
    rng = np.random.default_rng(9)
    # logits on a 1/256 grid, so adding 5 and dividing by 2 are exact in fp32
    x = (np.round(rng.standard_normal((3, 400)) * 3 * 256) / 256).astype(np.float32)
    _, lq, ent = oracle.expand_topk(x, 4, T)
    perm = rng.permutation(400)
    _, _, ent_p = oracle.expand_topk(x[:, perm], 4, T)
    _, lq_c, ent_c = oracle.expand_topk(x + np.float32(5.0), 4, T)
    np.testing.assert_allclose(ent_p, ent, rtol=1e-12)
    np.testing.assert_allclose(ent_c, ent, rtol=1e-9)
    np.testing.assert_allclose(lq_c, lq, atol=1e-9)
    # T scales the logits by 1/T (exact for powers of two)
    _, lq_s, ent_s = oracle.expand_topk((x / np.float32(T)).astype(np.float32), 4, 1.0)
    if T in (0.5, 2.0):
        np.testing.assert_allclose(ent_s, ent, rtol=1e-12)
        np.testing.assert_allclose(lq_s, lq, atol=1e-12)
    # log q of the tokens sum, with the rest, to probability one
    assert (np.exp(lq).sum(axis=1) <= 1 + 1e-12).all()


def test_neg_inf_logits_add_nothing_and_bad_rows_raise():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 100))).astype(np.float32)
    y = np.concatenate([x, np.full((2, 50), -np.inf, np.float32)], axis=1)
    t1, l1, e1 = oracle.expand_topk(x, 3)
    t2, l2, e2 = oracle.expand_topk(y, 3)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    np.testing.assert_allclose(e1, e2, rtol=1e-12)
    bad = x.copy()
    bad[1, 5] = np.nan
    with pytest.raises(ValueError):
        oracle.expand_topk(bad, 2)
    with pytest.raises(ValueError):
        oracle.expand_topk(np.full((1, 10), -np.inf, np.float32), 2)
    with pytest.raises(ValueError):
        oracle.expand_topk(x, 101)
