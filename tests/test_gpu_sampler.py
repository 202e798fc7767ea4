"""GPU parity: spec_verify_sample, its uniforms and its softmax against the oracle."""

import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import P_TOL, compare_walk, device, run_walk, say, walk_arrays
from synth import make_workload, random_parent
from synth.device import to_numpy

pytestmark = pytest.mark.gpu


def test_uniforms_match_oracle():
    say("sampler: uniforms")
    for seed, offset, B, N in [(0, 0, 8, 64), (12345, 77, 3, 256), (2**63 + 1, 2**40, 2, 5)]:
        u = to_numpy(tav.philox_uniforms(seed, offset, B, N, device=device()))
        ref = oracle.node_uniforms(seed, offset, B, N)
        np.testing.assert_array_equal(u.astype(np.float64), ref)


@pytest.mark.parametrize("V,T", [(1000, 1.0), (128256, 1.0), (151936, 0.7), (8, 1.3)])
def test_target_probs_match_oracle(V, T):
    say(f"sampler: target probs V={V} T={T}")
    rng = np.random.default_rng(V)
    logits = (rng.standard_normal((6, V)) * 3).astype(np.float32)
    logits[1, :V // 3] = -np.inf
    p = to_numpy(tav.target_probs(torch.from_numpy(logits).to(device()), T))
    ref = oracle.softmax(logits, T)
    # the device's all-fp64 softmax (not the walk's: see the probe test)
    assert np.abs(p - ref).max() <= 1e-12
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)


@pytest.mark.parametrize("name,T", [("llama70b", 1.0), ("llama70b", 0.7), ("long", 1.0),
                                    ("long", 0.7), ("llama8b", 1.3)])
def test_walk_softmax_matches_oracle(name, T):
    """The p and q the walk itself decides with (its fp32 per-entry
    exponentials, fp64 sums and rebases), at every visited node, against the
    oracle's fp64 softmax: within 1e-5, absolute and relative; and the p, q of
    each tested child's token likewise."""
    say(f"sampler: probe of the walk's softmax, {name} T={T}")
    w = make_workload(name, temperature=T)
    dev = device()
    from synth.device import upload
    d = upload(w, dev)
    flags = tav.new_flags(dev)
    path, n_acc, toks, p_rows, q_rows, cpq = tav.spec_verify_sample_probe(
        d["target_logits"], d["draft_logits"], d["parent"], d["token"], T, w.philox_seed,
        w.philox_offset, dev_flags=flags)
    path2, n_acc2, toks2 = tav.spec_verify_sample(
        d["target_logits"], d["draft_logits"], d["parent"], d["token"], T, w.philox_seed,
        w.philox_offset, dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    # the probe takes the same decisions as the walk it instruments
    assert torch.equal(path, path2) and torch.equal(n_acc, n_acc2) and torch.equal(toks, toks2)
    path, n_acc = to_numpy(path), to_numpy(n_acc)
    worst_abs = worst_rel = 0.0
    rows = 0
    for b in range(w.B):
        kids = set(int(x) for x in w.parent[b, 1:])
        for u in path[b, :n_acc[b] + 1]:
            u = int(u)
            for logits, got, need in ((w.target_logits[b, u], p_rows[b, u], True),
                                      (w.draft_logits[b, u], q_rows[b, u], u in kids)):
                if not need:
                    continue
                g = to_numpy(got)
                ref = oracle.softmax(logits, T)
                assert np.isfinite(g).all()
                err = np.abs(g - ref)
                worst_abs = max(worst_abs, float(err.max()))
                nz = ref > 0
                assert (g[~nz] == 0).all()
                worst_rel = max(worst_rel, float((err[nz] / ref[nz]).max()))
                rows += 1
            pu = oracle.softmax(w.target_logits[b, u], T)
            qu = oracle.softmax(w.draft_logits[b, u], T)
            for c in np.nonzero(w.parent[b] == u)[0]:
                if c == 0:
                    continue
                x = int(w.token[b, c])
                gp, gq = to_numpy(cpq[b, c])
                worst_abs = max(worst_abs, abs(gp - pu[x]), abs(gq - qu[x]))
                worst_rel = max(worst_rel, abs(gp - pu[x]) / pu[x], abs(gq - qu[x]) / qu[x])
    say(f"  {rows} rows, max abs {worst_abs:.2e}, max rel {worst_rel:.2e}")
    assert worst_abs <= P_TOL
    assert worst_rel <= P_TOL


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", dict(N=40, B=64, V=1000, tree="random", seed=5)),
    ("tiny", dict(N=256, B=4, V=3000, tree="random", seed=6)),
    ("tiny", dict(N=1, B=50, V=5000, tree="chain", seed=7)),
    ("tiny", dict(N=12, B=32, V=4097, tree="chain", seed=8, sigma_d=0.1)),
    ("tiny", dict(N=30, B=16, V=777, tree="random", temperature=0.6, seed=9)),
    ("llama8b", {}),
    ("llama70b", {}),
    ("long", {}),
    ("sweep_tree16", dict(B=16, accept=0.5)),
    ("sweep_chain6", dict(B=64, accept=0.8)),
])
def test_walk_matches_oracle(name, over):
    say(f"sampler: walk {name} {over}")
    w = make_workload(name, **over)
    path, n_acc, toks, flags = run_walk(w, device())
    assert flags == 0
    ref = oracle.verify_walk(w.target_logits, w.draft_logits, w.parent, w.token, w.temperature,
                             w.philox_seed, w.philox_offset)
    excused, draws = compare_walk(ref, path, n_acc, toks)
    say(f"  accepted {n_acc.tolist()[:8]}, excused {excused} of {draws} draws")


def test_walk_many_small_trees_and_offsets():
    rng = np.random.default_rng(11)
    B, N, V = 4096, 9, 64
    parent = np.stack([random_parent(rng, N) for _ in range(B)])
    tl = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    dl = (tl + rng.standard_normal((B, N, V)) * 0.7).astype(np.float32)
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    total_excused = total_draws = 0
    for offset in range(3):
        say(f"sampler: 4096 small trees, offset {offset}")
        path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 21, offset, device())
        assert flags == 0
        ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 21, offset)
        e, d = compare_walk(ref, path, n_acc, toks)
        total_excused += e
        total_draws += d
    assert total_excused <= 1e-4 * total_draws


def test_walk_is_deterministic():
    say("sampler: determinism")
    w = make_workload("tiny", N=40, B=64, V=20000, tree="random", seed=3)
    a = run_walk(w, device())
    b = run_walk(w, device())
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_chi_square_output_distribution_is_p_on_gpu():
    """10^6 trials, vocab 8, root with 3 leaf children drafted i.i.d. from q."""
    rng = np.random.default_rng(103)
    V, k, trials = 8, 3, 10**6
    pl = (rng.standard_normal(V) * 1.5).astype(np.float32)
    ql = (rng.standard_normal(V) * 1.5).astype(np.float32)
    q = scipy.special.softmax(ql.astype(np.float64))
    p = scipy.special.softmax(pl.astype(np.float64))
    tl = np.broadcast_to(pl, (trials, k + 1, V)).copy()
    dl = np.broadcast_to(ql, (trials, k + 1, V)).copy()
    parent = np.tile(np.array([-1] + [0] * k, np.int32), (trials, 1))
    token = np.zeros((trials, k + 1), np.int32)
    token[:, 1:] = rng.choice(V, size=(trials, k), p=q)
    say("sampler: chi-square 1e6 trials")
    path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 5, 0, device())
    assert flags == 0
    counts = np.bincount(toks[:, 0], minlength=V)
    stat = float(((counts - p * trials) ** 2 / (p * trials)).sum())
    assert stat < 24.32, stat
    ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 5, 0)
    compare_walk(ref, path, n_acc, toks)


def test_closed_form_on_gpu():
    gamma, alpha, trials = 5, 0.8, 10**6
    V, N = 8, gamma + 1
    pl = np.log(np.r_[[alpha / 4] * 4, [(1 - alpha) / 4] * 4]).astype(np.float32)
    ql = np.r_[[0.0] * 4, [-np.inf] * 4].astype(np.float32)
    tl = np.broadcast_to(pl, (trials, N, V)).copy()
    dl = np.broadcast_to(ql, (trials, N, V)).copy()
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (trials, 1))
    token = np.random.default_rng(4).integers(0, 4, (trials, N)).astype(np.int32)
    say("sampler: closed form gamma=5 alpha=0.8")
    path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 3, 1, device())
    assert flags == 0
    emitted = n_acc.astype(np.float64) + 1
    expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(emitted.mean() - expect) < 5 * emitted.std() / np.sqrt(trials)


def _zero_counters():
    path = os.path.join(os.path.dirname(__file__), "golden", "zero_uniforms.txt")
    found = {}
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            kind, seed, offset, node = line.split()
            found[kind] = (int(seed), int(offset), int(node))
    return found


def test_tie_rules_at_zero_uniforms():
    z = _zero_counters()
    say("sampler: zero-uniform tie rules")
    seed, off, _ = z["resample"]
    tl = np.array([[[-np.inf, -np.inf, 0.3, 1.0, -np.inf, 2.0, 0.0, 0.1]]], np.float32)
    _, _, toks, flags = walk_arrays(tl, tl, np.array([[-1]]), np.zeros((1, 1)), 1.0, seed, off,
                                    device())
    assert flags == 0 and toks[0, 0] == 2
    seed, off, node = z["acceptance"]
    dl = np.zeros((1, 2, 8), np.float32)
    tl = np.zeros((1, 2, 8), np.float32)
    tl[0, 0, 4] = -np.inf
    parent = np.array([[-1, 0]])
    _, n_acc, toks, _ = walk_arrays(tl, dl, parent, np.array([[0, 4]]), 1.0, seed, off, device())
    assert n_acc[0] == 0 and toks[0, 0] != 4
    _, n_acc, toks, _ = walk_arrays(tl, dl, parent, np.array([[0, 5]]), 1.0, seed, off, device())
    assert n_acc[0] == 1 and toks[0, 0] == 5


def test_flags_for_bad_inputs():
    say("sampler: bad-input flags")
    V = 50
    tl = np.zeros((3, 4, V), np.float32)
    parent = np.tile(np.array([-1, 0, 1, 0], np.int32), (3, 1))
    token = np.ones((3, 4), np.int32)
    t1 = tl.copy()
    t1[1, 0, 7] = np.nan
    *_, flags = walk_arrays(t1, tl, parent, token, 1.0, 0, 0, device())
    assert flags & tav.FLAG_NONFINITE_LOGITS
    t2 = tl.copy()
    t2[2, 0, :] = -np.inf
    *_, flags = walk_arrays(t2, tl, parent, token, 1.0, 0, 0, device())
    assert flags & tav.FLAG_NONFINITE_LOGITS
    p2 = parent.copy()
    p2[0, 3] = 3
    *_, flags = walk_arrays(tl, tl, p2, token, 1.0, 0, 0, device())
    assert flags & tav.FLAG_BAD_PARENT
    tk = token.copy()
    tk[1, 2] = V
    path, n_acc, toks, flags = walk_arrays(tl, tl, parent, tk, 1.0, 0, 0, device())
    assert flags & tav.FLAG_BAD_TOKEN
    # the good sequences in the batch still match the oracle
    ref = oracle.verify_walk(tl[[0, 2]], tl[[0, 2]], parent[[0, 2]], tk[[0, 2]], 1.0, 0, 0)
    # sequence indices feed the uniforms, so compare sequence 0 only
    assert (path[0] == ref.path[0]).all() and (toks[0] == ref.out_tokens[0]).all()
