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


def _scatter_tree(w):
    """The tree's rows at positions L..L+N-1, written by the pinned oracle commit."""
    ident = np.tile(np.arange(w.N, dtype=np.int32), (w.B, 1))
    full = np.full(w.B, w.N - 1, np.int32)
    k, v, _, _ = oracle.kv_commit(w.k_tree, w.v_tree, ident, full, w.block_table, w.prefix_len,
                                  w.k_cache, w.v_cache)
    return k, v


@pytest.mark.parametrize("cfg", [
    dict(N=5, B=1, D=64, Hkv=1, L=(128, 128)),
    dict(N=40, B=6, D=128, Hkv=8, L=(0, 50)),
    dict(N=64, B=8, D=128, Hkv=8, L=(6144, 8192)),
    dict(N=256, B=3, D=128, Hkv=4, L=(15, 17)),
    dict(N=200, B=3, D=64, Hkv=2, L=(1, 300)),
])
def test_inplace_commit_matches_oracle(cfg):
    say(f"commit in place: {cfg}")
    w = make_workload("tiny", tree="random", with_logits=False, Hq=cfg["Hkv"], seed=cfg["N"] + 1,
                      **cfg)
    path, n_acc = _random_paths(w, np.random.default_rng(2))
    k_c, v_c = _scatter_tree(w)
    dev = device()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kc, vc = t(k_c.view(np.int16)), t(v_c.view(np.int16))
    d = upload(w, dev, logits=False)
    flags = tav.new_flags(dev)
    slots, new_len = tav.kv_commit_inplace(t(path), t(n_acc), d["block_table"], d["prefix_len"],
                                           kc, vc, dev_flags=flags)
    torch.cuda.synchronize()
    k2, v2, ref_slots, ref_len = oracle.kv_commit_inplace(path, n_acc, w.block_table,
                                                          w.prefix_len, k_c, v_c)
    assert int(flags.item()) == 0
    np.testing.assert_array_equal(to_numpy(slots), ref_slots)
    np.testing.assert_array_equal(to_numpy(new_len), ref_len)
    np.testing.assert_array_equal(to_numpy(kc, np.uint16), k2)
    np.testing.assert_array_equal(to_numpy(vc, np.uint16), v2)


def test_inplace_commit_of_walk_paths_equals_the_copying_commit():
    # the sampler's own paths on the 70B-shaped batch: rolling back in place
    # leaves the accepted positions as the copying commit writes them
    say("commit in place: sampler paths, 70B-shaped batch")
    w = make_workload("llama70b")
    dev = device()
    d = upload(w, dev)
    flags = tav.new_flags(dev)
    path, n_acc, _ = tav.spec_verify_sample(d["target_logits"], d["draft_logits"], d["parent"],
                                            d["token"], 1.0, 0, 0, dev_flags=flags)
    k_c, v_c = _scatter_tree(w)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kc, vc = t(k_c.view(np.int16)), t(v_c.view(np.int16))
    s1, l1 = tav.kv_commit_inplace(path, n_acc, d["block_table"], d["prefix_len"], kc, vc,
                                   dev_flags=flags)
    s2, l2 = tav.kv_commit_path(d["k_tree"], d["v_tree"], path, n_acc, d["block_table"],
                                d["prefix_len"], d["k_cache"], d["v_cache"], dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert torch.equal(s1, s2) and torch.equal(l1, l2)
    slots = to_numpy(s1)
    kc_n, vc_n = to_numpy(kc, np.uint16), to_numpy(vc, np.uint16)
    k2, v2 = to_numpy(d["k_cache"], np.uint16), to_numpy(d["v_cache"], np.uint16)
    for b in range(w.B):
        for tt in range(int(to_numpy(n_acc)[b]) + 1):
            blk, s = divmod(int(slots[b, tt]), w.block)
            np.testing.assert_array_equal(kc_n[blk, :, s, :], k2[blk, :, s, :])
            np.testing.assert_array_equal(vc_n[blk, :, :, s], v2[blk, :, :, s])


def test_inplace_commit_of_a_root_chain_moves_nothing_and_short_tables_flag():
    say("commit in place: root chain, short table")
    w = make_workload("tiny", N=12, L=(30, 90), B=4, tree="chain", with_logits=False, seed=7)
    k_c, v_c = _scatter_tree(w)
    dev = device()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    n_acc = np.array([0, 3, 7, 11], np.int32)
    path = np.full((w.B, w.N), -1, np.int32)
    for b in range(w.B):
        path[b, :n_acc[b] + 1] = np.arange(n_acc[b] + 1)
    kc, vc = t(k_c.view(np.int16)), t(v_c.view(np.int16))
    d = upload(w, dev, logits=False)
    flags = tav.new_flags(dev)
    tav.kv_commit_inplace(t(path), t(n_acc), d["block_table"], d["prefix_len"], kc, vc,
                          dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    np.testing.assert_array_equal(to_numpy(kc, np.uint16), k_c)
    np.testing.assert_array_equal(to_numpy(vc, np.uint16), v_c)
    # a table that cannot hold the tree: flagged, nothing moves
    w2 = make_workload("tiny", N=5, L=(126, 126), with_logits=False, seed=0)
    d2 = upload(w2, dev, logits=False)
    table = d2["block_table"][:, :8].contiguous()
    before = d2["k_cache"].clone()
    flags = tav.new_flags(dev)
    slots, _ = tav.kv_commit_inplace(t(np.array([[0, 2, -1, -1, -1]], np.int32)),
                                     t(np.array([1], np.int32)), table, d2["prefix_len"],
                                     d2["k_cache"], d2["v_cache"], dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & tav.FLAG_CAPACITY
    assert (to_numpy(slots) == -1).all() and torch.equal(before, d2["k_cache"])
