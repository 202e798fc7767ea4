"""GPU parity of the fused walk-and-commit entry point: its outputs are the
bytes that spec_verify_sample (or its without-replacement or greedy form)
followed by kv_commit_path write for the same arguments, including after a
walk that raised a flag; and the fused step agrees with the oracle."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import compare_walk, device, say
from synth import make_workload
from synth.device import to_numpy, upload


pytestmark = pytest.mark.gpu


def _separate(w, d, kc, vc, mode, flags):
    if mode == "wor":
        fn, T = tav.spec_verify_sample_wor, w.temperature
    else:
        fn, T = tav.spec_verify_sample, (0.0 if mode == "greedy" else w.temperature)
    path, n_acc, toks = fn(d["target_logits"], d["draft_logits"], d["parent"], d["token"], T,
                           w.philox_seed, w.philox_offset, dev_flags=flags)
    slots, new_len = tav.kv_commit_path(d["k_tree"], d["v_tree"], path, n_acc, d["block_table"],
                                        d["prefix_len"], kc, vc, dev_flags=flags)
    return path, n_acc, toks, slots, new_len


def _fused(w, d, kc, vc, mode, flags):
    T = 0.0 if mode == "greedy" else w.temperature
    return tav.spec_verify_sample_commit(
        d["target_logits"], d["draft_logits"], d["parent"], d["token"], d["k_tree"],
        d["v_tree"], d["block_table"], d["prefix_len"], kc, vc, T, w.philox_seed,
        w.philox_offset, without_replacement=(mode == "wor"), dev_flags=flags)


def _both(w, d, dev, mode):
    caches = {}
    outs = {}
    for kind, fn in (("separate", _separate), ("fused", _fused)):
        kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
        flags = tav.new_flags(dev)
        res = fn(w, d, kc, vc, mode, flags)
        torch.cuda.synchronize()
        outs[kind] = [to_numpy(t) for t in res] + [int(flags.item())]
        caches[kind] = (to_numpy(kc, np.uint16), to_numpy(vc, np.uint16))
    return outs, caches


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", dict(N=40, B=5, Hq=8, Hkv=2, D=128, L=(10, 400), V=5000, tree="random", seed=1)),
    ("tiny", dict(N=17, B=3, Hq=4, Hkv=4, D=64, L=(0, 35), V=3000, tree="chain", seed=2)),
    ("llama8b", {}),
    ("llama70b", {}),
    ("sweep_tree16", dict(B=64)),
])
@pytest.mark.parametrize("mode", ["iid", "wor", "greedy"])
def test_sample_commit_writes_what_the_two_calls_write(name, over, mode):
    say(f"fused walk+commit: {name} {over} {mode}")
    w = make_workload(name, **over)
    dev = device()
    d = upload(w, dev)
    outs, caches = _both(w, d, dev, mode)
    labels = ("path", "n_accepted", "out_tokens", "commit_slots", "new_prefix_len", "flags")
    for lab, a, b in zip(labels, outs["separate"], outs["fused"]):
        np.testing.assert_array_equal(a, b, err_msg=lab)
    assert outs["fused"][-1] == 0
    np.testing.assert_array_equal(caches["separate"][0], caches["fused"][0])
    np.testing.assert_array_equal(caches["separate"][1], caches["fused"][1])
    say(f"  accepted {outs['fused'][1].tolist()[:8]}")


def test_sample_commit_after_a_flagged_walk():
    """A sequence with a bad parent: both forms raise the same flag and commit
    the same rows (the root's, for the bad sequence)."""
    w = make_workload("tiny", N=30, B=4, Hq=8, Hkv=2, D=128, L=(40, 90), V=2000,
                      tree="random", seed=5)
    w.parent[2, 7] = 9        # not below its own index
    dev = device()
    d = upload(w, dev)
    say("fused walk+commit: bad parent in sequence 2")
    outs, caches = _both(w, d, dev, "iid")
    for a, b in zip(outs["separate"], outs["fused"]):
        np.testing.assert_array_equal(a, b)
    assert outs["fused"][-1] & tav.FLAG_BAD_PARENT
    np.testing.assert_array_equal(caches["separate"][0], caches["fused"][0])
    np.testing.assert_array_equal(caches["separate"][1], caches["fused"][1])


def test_fused_step_matches_oracle():
    """mask, attention, then the fused walk and commit, chained on one stream,
    against the oracle's composed step."""
    w = make_workload("tiny", N=48, B=6, Hq=16, Hkv=4, D=128, L=(100, 700), V=8000,
                      tree="random", seed=9)
    dev = device()
    d = upload(w, dev)
    say("fused step vs oracle")
    flags = tav.new_flags(dev)
    mask, _ = tav.tree_mask_build(d["parent"], dev_flags=flags)
    tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                         d["block_table"], d["prefix_len"], w.max_prefix_len, mask,
                         scale=w.scale, dev_flags=flags)
    path, n_acc, toks, slots, new_len = tav.spec_verify_sample_commit(
        d["target_logits"], d["draft_logits"], d["parent"], d["token"], d["k_tree"],
        d["v_tree"], d["block_table"], d["prefix_len"], d["k_cache"], d["v_cache"],
        w.temperature, w.philox_seed, w.philox_offset, dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    ref = oracle.verify_step_ref(w)
    path, n_acc, toks = to_numpy(path), to_numpy(n_acc), to_numpy(toks)
    compare_walk(ref.walk, path, n_acc, toks)
    k_ref, v_ref, s_ref, l_ref = oracle.kv_commit(w.k_tree, w.v_tree, path, n_acc,
                                                  w.block_table, w.prefix_len, w.k_cache,
                                                  w.v_cache)
    np.testing.assert_array_equal(to_numpy(slots), s_ref)
    np.testing.assert_array_equal(to_numpy(new_len), l_ref)
    np.testing.assert_array_equal(to_numpy(d["k_cache"], np.uint16), k_ref)
    np.testing.assert_array_equal(to_numpy(d["v_cache"], np.uint16), v_ref)


ATTN_CASES = [
    dict(N=5, B=1, Hq=1, Hkv=1, D=64, L=(128, 128), tree="example"),
    dict(N=40, B=3, Hq=8, Hkv=2, D=128, L=(1, 250), tree="random"),
    dict(N=64, B=2, Hq=64, Hkv=8, D=128, L=(500, 700), tree="random"),     # 2 row blocks
    dict(N=130, B=1, Hq=8, Hkv=4, D=64, L=(70, 70), tree="random"),        # 3 tree tiles
    dict(N=256, B=1, Hq=2, Hkv=1, D=128, L=(3000, 3000), tree="random"),   # 4 tree tiles, split-K
    dict(N=48, B=1, Hq=64, Hkv=8, D=64, L=(513, 700), tree="random"),
    dict(N=20, B=2, Hq=8, Hkv=2, D=128, L=(1000, 1100), tree="chain"),
]


@pytest.mark.parametrize("cfg", ATTN_CASES, ids=lambda c: f"N{c['N']}-G{c['Hq']//c['Hkv']}-D{c['D']}")
def test_attention_from_parents_is_the_mask_path(cfg):
    """tree_attn_verify_tree gives the bytes of tree_mask_build followed by
    tree_attn_verify, and writes the same mask and depths."""
    say(f"attention from parents: {cfg}")
    w = make_workload("tiny", with_logits=False, seed=cfg["N"] + 7, **cfg)
    dev = device()
    d = upload(w, dev, logits=False)
    f1, f2 = tav.new_flags(dev), tav.new_flags(dev)
    mask, depth = tav.tree_mask_build(d["parent"], dev_flags=f1)
    ref = tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                               d["block_table"], d["prefix_len"], w.max_prefix_len, mask,
                               scale=w.scale, dev_flags=f1)
    mask2 = torch.zeros_like(mask)
    depth2 = torch.full_like(depth, -7)
    out = tav.tree_attn_verify_tree(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                                    d["block_table"], d["prefix_len"], w.max_prefix_len,
                                    d["parent"], scale=w.scale, mask_out=mask2, depth_out=depth2,
                                    dev_flags=f2)
    torch.cuda.synchronize()
    assert int(f1.item()) == int(f2.item()) == 0
    np.testing.assert_array_equal(to_numpy(out).view(np.uint32), to_numpy(ref).view(np.uint32))
    np.testing.assert_array_equal(to_numpy(mask2, np.uint64), to_numpy(mask, np.uint64))
    np.testing.assert_array_equal(to_numpy(depth2), to_numpy(depth))


def test_attention_from_parents_with_prefix_lengths_far_apart():
    """Prefix lengths far apart under a split plan (some splits hold no
    tile): the built masks and depths are written once per sequence, and the
    output is the mask path's."""
    w = make_workload("tiny", with_logits=False, seed=12, B=6, N=70, Hq=16, Hkv=4, D=128,
                      L=(3000, 3000), tree="random")
    w.prefix_len[:] = [0, 3000, 7, 0, 1200, 64]
    dev = device()
    d = upload(w, dev, logits=False)
    say("attention from parents: prefix lengths far apart, split plan")
    f1, f2 = tav.new_flags(dev), tav.new_flags(dev)
    mask, depth = tav.tree_mask_build(d["parent"], dev_flags=f1)
    ref = tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                               d["block_table"], d["prefix_len"], 3000, mask, scale=w.scale,
                               dev_flags=f1)
    mask2 = torch.zeros_like(mask)
    depth2 = torch.full_like(depth, -7)
    out = tav.tree_attn_verify_tree(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                                    d["block_table"], d["prefix_len"], 3000, d["parent"],
                                    scale=w.scale, mask_out=mask2, depth_out=depth2, dev_flags=f2)
    torch.cuda.synchronize()
    assert int(f1.item()) == int(f2.item()) == 0
    np.testing.assert_array_equal(to_numpy(out).view(np.uint32), to_numpy(ref).view(np.uint32))
    np.testing.assert_array_equal(to_numpy(mask2, np.uint64), to_numpy(mask, np.uint64))
    np.testing.assert_array_equal(to_numpy(depth2), to_numpy(depth))


def test_attention_from_parents_flags_a_bad_tree_like_the_mask_builder():
    w = make_workload("tiny", with_logits=False, N=30, B=3, Hq=8, Hkv=2, D=128, L=(40, 90),
                      tree="random", seed=3)
    w.parent[1, 11] = 11
    dev = device()
    d = upload(w, dev, logits=False)
    say("attention from parents: bad parent")
    f1, f2 = tav.new_flags(dev), tav.new_flags(dev)
    mask, depth = tav.tree_mask_build(d["parent"], dev_flags=f1)
    mask2 = torch.zeros_like(mask)
    depth2 = torch.zeros_like(depth)
    tav.tree_attn_verify_tree(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                              d["block_table"], d["prefix_len"], w.max_prefix_len, d["parent"],
                              scale=w.scale, mask_out=mask2, depth_out=depth2, dev_flags=f2)
    torch.cuda.synchronize()
    assert int(f1.item()) == int(f2.item()) == tav.FLAG_BAD_PARENT
    np.testing.assert_array_equal(to_numpy(mask2, np.uint64), to_numpy(mask, np.uint64))
    np.testing.assert_array_equal(to_numpy(depth2), to_numpy(depth))
