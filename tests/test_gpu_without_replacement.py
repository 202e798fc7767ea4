"""GPU parity: spec_verify_sample_wor (siblings drawn from q without
replacement; a rejected token leaves q before the next sibling) against the
oracle's walk under the same rule."""

import numpy as np
import pytest
import scipy.special

import oracle
from gpu_helpers import compare_walk, device, run_walk, say, walk_arrays
from synth import make_workload, random_parent

pytestmark = pytest.mark.gpu


def _wor_tokens(rng, dl, parent):
    """Children of each node drawn from its draft row without replacement
    (the largest of log q + Gumbel noise, in child order)."""
    B, N, V = dl.shape
    token = np.zeros((B, N), np.int32)
    for b in range(B):
        for u in range(N):
            kids = np.nonzero(parent[b] == u)[0]
            if kids.size == 0:
                continue
            q = scipy.special.softmax(dl[b, u].astype(np.float64))
            with np.errstate(divide="ignore"):
                keys = np.log(q) + rng.gumbel(size=V)
            token[b, kids] = np.argsort(-keys, kind="stable")[:kids.size]
    return token


@pytest.mark.parametrize("name,over", [
    ("tiny", dict(N=40, B=64, V=1000, tree="random", seed=5)),
    ("tiny", dict(N=256, B=4, V=3000, tree="random", seed=6)),
    ("tiny", dict(N=30, B=16, V=777, tree="random", temperature=0.6, seed=9)),
    ("llama8b", {}),
    ("llama70b", {}),
    ("long", {}),
    ("sweep_tree16", dict(B=16, accept=0.5)),
])
def test_walk_matches_oracle(name, over):
    say(f"sampler wor: walk {name} {over}")
    w = make_workload(name, **over)
    path, n_acc, toks, flags = run_walk(w, device(), wor=True)
    assert flags == 0
    ref = oracle.verify_walk(w.target_logits, w.draft_logits, w.parent, w.token, w.temperature,
                             w.philox_seed, w.philox_offset, without_replacement=True)
    excused, draws = compare_walk(ref, path, n_acc, toks)
    say(f"  accepted {n_acc.tolist()[:8]}, excused {excused} of {draws} draws")


def test_many_small_trees_drafted_without_replacement():
    rng = np.random.default_rng(12)
    B, N, V = 4096, 9, 64
    parent = np.stack([random_parent(rng, N) for _ in range(B)])
    tl = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    dl = (tl + rng.standard_normal((B, N, V)) * 0.7).astype(np.float32)
    token = _wor_tokens(rng, dl, parent)
    total_excused = total_draws = differ = 0
    for offset in range(3):
        say(f"sampler wor: 4096 small trees, offset {offset}")
        path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 21, offset, device(),
                                               wor=True)
        assert flags == 0
        ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 21, offset,
                                 without_replacement=True)
        e, d = compare_walk(ref, path, n_acc, toks)
        total_excused += e
        total_draws += d
        iid = oracle.verify_walk(tl, dl, parent, token, 1.0, 21, offset)
        differ += int((iid.out_tokens != ref.out_tokens).any(axis=1).sum())
    assert total_excused <= 1e-4 * total_draws
    assert differ > 0   # the inputs do reach the point where the rules part


def test_chains_match_the_iid_entry_point():
    say("sampler wor: chains equal the i.i.d. rule")
    w = make_workload("tiny", N=12, B=64, V=4097, tree="chain", seed=8)
    a = run_walk(w, device())
    b = run_walk(w, device(), wor=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_is_deterministic():
    say("sampler wor: determinism")
    w = make_workload("tiny", N=40, B=64, V=20000, tree="random", seed=3)
    a = run_walk(w, device(), wor=True)
    b = run_walk(w, device(), wor=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_chi_square_output_distribution_is_p_on_gpu():
    """10^6 trials, vocabulary 8, root with 3 leaf children drafted from q
    without replacement."""
    rng = np.random.default_rng(104)
    V, k, trials = 8, 3, 10**6
    pl = rng.standard_normal(V).astype(np.float32)
    ql = np.r_[[3.0], rng.standard_normal(V - 1)].astype(np.float32)
    q = scipy.special.softmax(ql.astype(np.float64))
    p = scipy.special.softmax(pl.astype(np.float64))
    tl = np.broadcast_to(pl, (trials, k + 1, V)).copy()
    dl = np.broadcast_to(ql, (trials, k + 1, V)).copy()
    parent = np.tile(np.array([-1] + [0] * k, np.int32), (trials, 1))
    token = np.zeros((trials, k + 1), np.int32)
    keys = np.log(q)[None, :] + rng.gumbel(size=(trials, V))
    token[:, 1:] = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    say("sampler wor: chi-square 1e6 trials")
    path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 6, 0, device(), wor=True)
    assert flags == 0
    counts = np.bincount(toks[:, 0], minlength=V)
    stat = float(((counts - p * trials) ** 2 / (p * trials)).sum())
    assert stat < 24.32, stat
    ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 6, 0, without_replacement=True)
    compare_walk(ref, path, n_acc, toks)


def test_every_token_drafted_accepts_one():
    """V = 2 with both tokens as children of the root: one is always accepted."""
    rng = np.random.default_rng(13)
    B, V = 4000, 2
    tl = np.zeros((B, 3, V), np.float32)
    dl = np.zeros((B, 3, V), np.float32)
    tl[:, 0] = rng.standard_normal((B, V)) * 2
    dl[:, 0] = rng.standard_normal((B, V)) * 2
    parent = np.tile(np.array([-1, 0, 0], np.int32), (B, 1))
    token = np.zeros((B, 3), np.int32)
    token[:, 1] = rng.integers(0, 2, B)
    token[:, 2] = 1 - token[:, 1]
    say("sampler wor: both tokens drafted")
    path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 8, 0, device(), wor=True)
    assert flags == 0
    assert (n_acc == 1).all()
    ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 8, 0, without_replacement=True)
    compare_walk(ref, path, n_acc, toks)
