"""GPU parity of the walk at batches larger than the device holds groups
for (spec_verify_sample and spec_verify_sample_wor): every group then walks
several sequences in turn, so these cases cover a group's second and later
sequences (state reset between them, the mailbox generations carried on,
the fused commit after each) under both sibling rules, with one and several
workgroups per sequence, many rejections, ragged chunks, determinism and the
input flags. Most take the layout with 28 entries per thread (16 held in
registers, 12 in LDS, fetched ahead by direct loads; rows that are not
16-byte aligned go through registers instead); one takes 16 per thread."""

import dataclasses

import numpy as np
import pytest

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import compare_walk, device, run_walk, say, walk_arrays
from synth import make_workload, random_parent
from synth.device import to_numpy, upload

pytestmark = pytest.mark.gpu


def _in_turn(B, V, least=3, entries=None):
    plan = tav.sampler_plan(B, V)
    say(f"  plan {plan}")
    assert plan["sequences_per_group"] >= least
    if entries is not None:
        assert plan["entries_per_thread"] == entries
    return plan


# Vocabularies above 8192 entries take several workgroups per sequence, so
# these batches leave two or more sequences per group. (Layouts as a
# 256-CU device plans them.)
CASES = [
    # (workload, overrides, workgroups per sequence at least, sequences per
    #  group at least, entries per thread)
    ("tiny", dict(N=8, B=300, V=28000, tree="random", seed=31), 2, 3, 28),   # ragged last step and chunk
    ("tiny", dict(N=8, B=200, V=43000, tree="random", seed=32), 3, 3, 28),
    ("tiny", dict(N=8, B=200, V=43000, tree="chain", seed=33, sigma_d=3.0), 3, 3, 28),   # many rejections
    ("tiny", dict(N=16, B=300, V=28001, tree="random", temperature=0.6, seed=34), 2, 3, 28),   # odd V: no 16-byte loads
    ("tiny", dict(N=8, B=70, V=50000, tree="random", seed=36), 7, 2, 16),   # registers only
    ("sweep_tree16", dict(B=64, accept=0.5), 16, 4, 16),
    ("sweep_chain6", dict(B=128, accept=0.9), 9, 5, 28),
]


@pytest.mark.parametrize("wor", [False, True], ids=["iid", "wor"])
@pytest.mark.parametrize("name,over,members,least,entries", CASES,
                         ids=lambda c: str(c)[:40] if isinstance(c, dict) else None)
def test_walk_in_turn_matches_oracle(name, over, members, least, entries, wor):
    say(f"walk, sequences in turn: {name} {over} wor={wor}")
    w = make_workload(name, **over)
    plan = _in_turn(w.B, w.V, least, entries)
    assert plan["workgroups_per_sequence"] >= members
    path, n_acc, toks, flags = run_walk(w, device(), wor=wor)
    assert flags == 0
    ref = oracle.verify_walk(w.target_logits, w.draft_logits, w.parent, w.token, w.temperature,
                             w.philox_seed, w.philox_offset, without_replacement=wor)
    excused, draws = compare_walk(ref, path, n_acc, toks)
    say(f"  accepted {n_acc.tolist()[:8]}, excused {excused} of {draws} draws")


def test_walk_in_turn_many_offsets():
    """300 sequences of 6-node random trees over a 28004-token vocabulary
    (two workgroups per sequence, chunks of 14004 and 14000 entries that end
    inside the last run of their LDS entries), five Philox offsets. (The
    oracle's draws here stay 3e-8 or more from their boundaries.)"""
    rng = np.random.default_rng(41)
    B, N, V = 300, 6, 28004
    parent = np.stack([random_parent(rng, N) for _ in range(B)])
    tl = (rng.standard_normal((B, N, V)) * 2.0).astype(np.float32)
    dl = (tl + rng.standard_normal((B, N, V)) * 1.0).astype(np.float32)
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    plan = _in_turn(B, V, least=2, entries=28)
    assert plan["workgroups_per_sequence"] == 2
    total_excused = total_draws = 0
    for offset in range(5):
        say(f"walk in turn: offset {offset}")
        path, n_acc, toks, flags = walk_arrays(tl, dl, parent, token, 1.0, 5, offset, device())
        assert flags == 0
        ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 5, offset)
        e, d = compare_walk(ref, path, n_acc, toks)
        total_excused += e
        total_draws += d
    assert total_excused <= 1e-4 * total_draws


def test_walk_in_turn_is_deterministic():
    w = make_workload("tiny", N=8, B=128, V=50000, tree="random", seed=35)
    _in_turn(w.B, w.V, least=2)
    say("walk in turn: determinism")
    a = run_walk(w, device())
    b = run_walk(w, device())
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_walk_in_turn_flags_bad_inputs():
    """A NaN logit (in a register entry, and in an LDS entry), a row of
    -inf, a bad parent and a bad token, in sequences a group walks after
    others, each raise their flag and fail only their own sequence."""
    rng = np.random.default_rng(42)
    B, N, V = 520, 4, 9000
    tl = (rng.standard_normal((B, N, V))).astype(np.float32)
    parent = np.tile(np.array([-1, 0, 1, 0], np.int32), (B, 1))
    token = rng.integers(0, V, (B, N)).astype(np.int32)
    _in_turn(B, V, least=2, entries=28)
    say("walk in turn: bad-input flags")
    t1 = tl.copy()
    t1[1, 0, 4097] = np.nan
    path, n_acc, toks, flags = walk_arrays(t1, tl, parent, token, 1.0, 0, 0, device())
    assert flags == tav.FLAG_NONFINITE_LOGITS
    assert n_acc[1] == 0 and (path[1, 1:] == -1).all() and (toks[1] == -1).all()
    t1 = tl.copy()
    t1[1, 0, 8500] = np.nan   # past the 8192 register entries of the one workgroup
    path, n_acc, toks, flags = walk_arrays(t1, tl, parent, token, 1.0, 0, 0, device())
    assert flags == tav.FLAG_NONFINITE_LOGITS
    assert n_acc[1] == 0 and (path[1, 1:] == -1).all() and (toks[1] == -1).all()
    t2 = tl.copy()
    t2[2, 0, :] = -np.inf
    *_, flags = walk_arrays(t2, tl, parent, token, 1.0, 0, 0, device())
    assert flags == tav.FLAG_NONFINITE_LOGITS
    p2 = parent.copy()
    p2[0, 3] = 3
    *_, flags = walk_arrays(tl, tl, p2, token, 1.0, 0, 0, device())
    assert flags == tav.FLAG_BAD_PARENT
    tk = token.copy()
    tk[1, 2] = V
    path, n_acc, toks, flags = walk_arrays(tl, tl, parent, tk, 1.0, 0, 0, device())
    assert flags == tav.FLAG_BAD_TOKEN
    assert n_acc[1] == 0 and (toks[1] == -1).all()
    # every other sequence still matches the oracle
    ref = oracle.verify_walk(tl, tl, parent, token, 1.0, 0, 0)
    keep = np.arange(B) != 1
    sub = dataclasses.replace(ref, **{f.name: getattr(ref, f.name)[keep]
                                      for f in dataclasses.fields(ref)
                                      if isinstance(getattr(ref, f.name), np.ndarray)})
    compare_walk(sub, path[keep], n_acc[keep], toks[keep])


@pytest.mark.parametrize("wor", [False, True], ids=["iid", "wor"])
def test_fused_commit_in_turn_matches_separate_calls(wor):
    """spec_verify_sample_commit with groups walking several sequences in
    turn writes what the walk followed by kv_commit_path writes."""
    w = make_workload("sweep_tree16", B=128, accept=0.8)
    _in_turn(w.B, w.V)
    dev = device()
    d = upload(w, dev)
    say(f"walk in turn: fused commit, wor={wor}")
    outs = {}
    for kind in ("separate", "fused"):
        kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
        flags = tav.new_flags(dev)
        if kind == "separate":
            fn = tav.spec_verify_sample_wor if wor else tav.spec_verify_sample
            path, n_acc, toks = fn(d["target_logits"], d["draft_logits"], d["parent"], d["token"],
                                   w.temperature, w.philox_seed, w.philox_offset, dev_flags=flags)
            slots, new_len = tav.kv_commit_path(d["k_tree"], d["v_tree"], path, n_acc,
                                                d["block_table"], d["prefix_len"], kc, vc,
                                                dev_flags=flags)
            res = (path, n_acc, toks, slots, new_len)
        else:
            res = tav.spec_verify_sample_commit(
                d["target_logits"], d["draft_logits"], d["parent"], d["token"], d["k_tree"],
                d["v_tree"], d["block_table"], d["prefix_len"], kc, vc, w.temperature,
                w.philox_seed, w.philox_offset, without_replacement=wor, dev_flags=flags)
        torch_sync()
        outs[kind] = [to_numpy(t) for t in res] + [int(flags.item()),
                                                  to_numpy(kc, np.uint16), to_numpy(vc, np.uint16)]
    for a, b in zip(outs["separate"], outs["fused"]):
        np.testing.assert_array_equal(a, b)
    assert outs["fused"][5] == 0


def torch_sync():
    import torch
    torch.cuda.synchronize()
