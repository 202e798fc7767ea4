"""Pins of the oracle's greedy (temperature 0) verification.

LLM Primer VI ch. 9, section 9.1: the longest prefix of candidates matching
the target's own choice is accepted, and at the first mismatch the engine
commits to the target's choice. These tests check that statement on chains,
the sibling order on trees, and the low-temperature limit of the stochastic
walk (pinned separately) on chains of top-1 draft tokens.
"""

import numpy as np
import pytest

import oracle


def _logits(rng, B, N, V, scale=3.0):
    return (rng.standard_normal((B, N, V)) * scale).astype(np.float32)


def _chain(N):
    return np.arange(-1, N - 1, dtype=np.int32)


@pytest.mark.parametrize("N", [1, 2, 7, 40])
def test_fully_matching_chain_is_accepted_to_the_end(N):
    rng = np.random.default_rng(N)
    B, V = 3, 50
    tl = _logits(rng, B, N, V)
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = tl[:, :-1].argmax(axis=2)          # node i carries row i-1's choice
    r = oracle.verify_greedy(tl, np.tile(_chain(N), (B, 1)), tok)
    assert (r.n_accepted == N - 1).all()
    np.testing.assert_array_equal(r.path, np.tile(np.arange(N), (B, 1)))
    # emitted: the accepted tokens, then the leaf's own choice (the bonus)
    np.testing.assert_array_equal(r.out_tokens[:, :N - 1], tok[:, 1:])
    np.testing.assert_array_equal(r.out_tokens[:, N - 1], tl[:, N - 1].argmax(axis=1))


@pytest.mark.parametrize("k", [0, 1, 3, 6])
def test_longest_matching_prefix_then_the_targets_choice(k):
    rng = np.random.default_rng(10 + k)
    B, N, V = 4, 8, 30
    tl = _logits(rng, B, N, V)
    choice = tl.argmax(axis=2)
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = choice[:, :-1]
    # first mismatch at node k + 1 (any other token), later nodes arbitrary
    tok[:, k + 1] = (choice[:, k] + 1) % V
    tok[:, k + 2:] = rng.integers(0, V, size=(B, N - k - 2))
    r = oracle.verify_greedy(tl, np.tile(_chain(N), (B, 1)), tok)
    assert (r.n_accepted == k).all()
    np.testing.assert_array_equal(r.out_tokens[:, :k], tok[:, 1:k + 1])
    np.testing.assert_array_equal(r.out_tokens[:, k], choice[:, k])
    assert (r.out_tokens[:, k + 1:] == -1).all() and (r.path[:, k + 1:] == -1).all()


def test_siblings_are_scanned_in_order_and_duplicates_take_the_lower_index():
    V = 10
    tl = np.zeros((1, 5, V), np.float32)
    tl[0, 0, 7] = 5.0          # root's choice: 7
    tl[0, 2, 3] = 4.0          # node 2's choice: 3
    tl[0, 4, 9] = 1.0
    parent = np.array([[-1, 0, 0, 0, 2]], np.int32)
    token = np.array([[0, 1, 7, 7, 3]], np.int32)   # nodes 2 and 3 both carry 7
    r = oracle.verify_greedy(tl, parent, token)
    assert r.n_accepted[0] == 2
    np.testing.assert_array_equal(r.path[0, :3], [0, 2, 4])
    np.testing.assert_array_equal(r.out_tokens[0, :3], [7, 3, 9])


def test_ties_in_the_target_row_take_the_lowest_token():
    tl = np.zeros((1, 2, 6), np.float32)
    tl[0, 0, [2, 4]] = 1.0
    r = oracle.verify_greedy(tl, np.array([[-1, 0]]), np.array([[0, 4]]))
    assert r.n_accepted[0] == 0 and r.out_tokens[0, 0] == 2


@pytest.mark.parametrize("seed", range(6))
def test_low_temperature_limit_of_the_stochastic_walk_on_chains(seed):
    # chains of top-1 draft tokens: at T -> 0 the target and draft
    # distributions are one-hot, so min(1, p/q) accepts exactly the target's
    # choice and the residual is the target's choice
    rng = np.random.default_rng(100 + seed)
    B, N, V = 16, 6, 200
    tl = _logits(rng, B, N, V)
    dl = tl + (rng.standard_normal((B, N, V)) * 1.0).astype(np.float32)
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = dl[:, :-1].argmax(axis=2)
    par = np.tile(_chain(N), (B, 1))
    g = oracle.verify_greedy(tl, par, tok)
    s = oracle.verify_walk(tl, dl, par, tok, temperature=1e-4, seed=seed)
    np.testing.assert_array_equal(g.n_accepted, s.n_accepted)
    np.testing.assert_array_equal(g.path, s.path)
    np.testing.assert_array_equal(g.out_tokens, s.out_tokens)


def test_greedy_invalid_inputs_raise():
    tl = np.zeros((1, 3, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.verify_greedy(tl, np.array([[-1, 2, 0]]), np.array([[0, 1, 1]]))
    with pytest.raises(ValueError):
        oracle.verify_greedy(tl, np.array([[-1, 0, 0]]), np.array([[0, 1, 4]]))
    bad = tl.copy()
    bad[0, 0, 1] = np.nan
    with pytest.raises(ValueError):
        oracle.verify_greedy(bad, np.array([[-1, 0, 0]]), np.array([[0, 1, 1]]))
    bad = np.full((1, 3, 4), -np.inf, np.float32)
    with pytest.raises(ValueError):
        oracle.verify_greedy(bad, np.array([[-1, 0, 0]]), np.array([[0, 1, 1]]))
