"""GPU parity: tree_mask_build and kv_commit_path against the oracle (bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import device, run_mask, say
from synth import chain_parent, make_workload, random_parent
from synth.device import to_numpy, upload

pytestmark = pytest.mark.gpu


def _parents_workload(parents):
    w = make_workload("tiny", N=parents.shape[1], B=parents.shape[0], tree="chain",
                      with_logits=False, L=(0, 0))
    w.parent = parents.astype(np.int32)
    return w


def test_mask_worked_example():
    say("mask: worked example")
    mask, depth, flags = run_mask(make_workload("tiny", with_logits=False), device())
    assert flags == 0
    assert mask[0, :, 0].tolist() == [1, 3, 7, 9, 25]
    assert depth[0].tolist() == [0, 1, 2, 1, 2]


@pytest.mark.parametrize("N", [1, 2, 5, 63, 64, 65, 127, 128, 129, 200, 256])
def test_mask_matches_oracle(N):
    say(f"mask: N={N}")
    rng = np.random.default_rng(N)
    parents = np.stack([chain_parent(N)] + [random_parent(rng, N) for _ in range(63)])
    mask, depth, flags = run_mask(_parents_workload(parents), device())
    ref_mask, ref_depth = oracle.tree_mask(parents)
    assert flags == 0
    np.testing.assert_array_equal(mask, ref_mask)
    np.testing.assert_array_equal(depth, ref_depth)


def test_mask_ten_thousand_random_trees():
    rng = np.random.default_rng(99)
    total = 0
    for N in (3, 17, 64, 100, 256):
        say(f"mask: 2000 random trees N={N}")
        parents = np.stack([random_parent(rng, N) for _ in range(2000)])
        mask, depth, flags = run_mask(_parents_workload(parents), device())
        ref_mask, ref_depth = oracle.tree_mask(parents)
        assert flags == 0
        np.testing.assert_array_equal(mask, ref_mask)
        np.testing.assert_array_equal(depth, ref_depth)
        total += parents.shape[0]
    assert total == 10000


def test_mask_flags_bad_parent():
    say("mask: bad parent flag")
    rng = np.random.default_rng(5)
    parents = np.stack([random_parent(rng, 20) for _ in range(4)])
    parents[2, 7] = 9          # a later node as parent
    mask, depth, flags = run_mask(_parents_workload(parents), device())
    assert flags & tav.FLAG_BAD_PARENT
    good = [0, 1, 3]
    ref_mask, _ = oracle.tree_mask(parents[good])
    np.testing.assert_array_equal(mask[good], ref_mask)


def _random_paths(w, rng):
    B, N = w.parent.shape
    path = np.full((B, N), -1, np.int32)
    n_acc = np.zeros(B, np.int32)
    for b in range(B):
        u, p = 0, [0]
        while True:
            kids = [c for c in range(N) if w.parent[b, c] == u]
            if not kids or rng.random() < 0.15:
                break
            u = int(rng.choice(kids))
            p.append(u)
        path[b, :len(p)] = p
        n_acc[b] = len(p) - 1
    return path, n_acc


@pytest.mark.parametrize("cfg", [
    dict(N=5, B=1, D=64, Hkv=1, L=(128, 128)),
    dict(N=40, B=6, D=128, Hkv=8, L=(0, 50)),
    dict(N=64, B=8, D=128, Hkv=8, L=(6144, 8192)),
    dict(N=200, B=3, D=64, Hkv=2, L=(15, 17)),
])
def test_commit_matches_oracle(cfg):
    say(f"commit: {cfg}")
    w = make_workload("tiny", tree="random", with_logits=False, Hq=cfg["Hkv"], seed=cfg["N"],
                      **cfg)
    rng = np.random.default_rng(1)
    path, n_acc = _random_paths(w, rng)
    dev = device()
    d = upload(w, dev, logits=False)
    flags = tav.new_flags(dev)
    slots, new_len = tav.kv_commit_path(d["k_tree"], d["v_tree"],
                                        torch.from_numpy(path).to(dev),
                                        torch.from_numpy(n_acc).to(dev), d["block_table"],
                                        d["prefix_len"], d["k_cache"], d["v_cache"],
                                        dev_flags=flags)
    torch.cuda.synchronize()
    k2, v2, ref_slots, ref_len = oracle.kv_commit(w.k_tree, w.v_tree, path, n_acc, w.block_table,
                                                  w.prefix_len, w.k_cache, w.v_cache)
    assert int(flags.item()) == 0
    np.testing.assert_array_equal(to_numpy(slots), ref_slots)
    np.testing.assert_array_equal(to_numpy(new_len), ref_len)
    np.testing.assert_array_equal(to_numpy(d["k_cache"], np.uint16), k2)
    np.testing.assert_array_equal(to_numpy(d["v_cache"], np.uint16), v2)


def test_commit_flags_short_table_without_writing_past_it():
    say("commit: short table flag")
    w = make_workload("tiny", N=5, L=(128, 128), with_logits=False, seed=0)
    dev = device()
    d = upload(w, dev, logits=False)
    table = d["block_table"][:, :8].contiguous()       # room for exactly 128 tokens
    before_k = d["k_cache"].clone()
    flags = tav.new_flags(dev)
    path = torch.tensor([[0, 1, 2, -1, -1]], dtype=torch.int32, device=dev)
    n_acc = torch.tensor([2], dtype=torch.int32, device=dev)
    slots, new_len = tav.kv_commit_path(d["k_tree"], d["v_tree"], path, n_acc, table,
                                        d["prefix_len"], d["k_cache"], d["v_cache"],
                                        dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & tav.FLAG_CAPACITY
    assert (to_numpy(slots) == -1).all()
    assert torch.equal(before_k, d["k_cache"])
