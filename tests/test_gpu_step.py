"""GPU parity of the whole verification step: the four calls chained on one
stream with no host synchronisation, against the oracle's composed step."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import ATTN_TOL, compare_walk, device, say
from synth import make_workload
from synth.device import to_numpy, upload


pytestmark = pytest.mark.gpu


def _step(w, d, dev):
    flags = tav.new_flags(dev)
    mask, depth = tav.tree_mask_build(d["parent"], dev_flags=flags)
    out = tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                               d["block_table"], d["prefix_len"], w.max_prefix_len, mask,
                               scale=w.scale, dev_flags=flags)
    path, n_acc, toks = tav.spec_verify_sample(d["target_logits"], d["draft_logits"],
                                               d["parent"], d["token"], w.temperature,
                                               w.philox_seed, w.philox_offset, dev_flags=flags)
    slots, new_len = tav.kv_commit_path(d["k_tree"], d["v_tree"], path, n_acc,
                                        d["block_table"], d["prefix_len"], d["k_cache"],
                                        d["v_cache"], dev_flags=flags)
    torch.cuda.synchronize()
    return dict(mask=to_numpy(mask, np.uint64), depth=to_numpy(depth), out=to_numpy(out),
                path=to_numpy(path), n_acc=to_numpy(n_acc), toks=to_numpy(toks),
                slots=to_numpy(slots), new_len=to_numpy(new_len), flags=int(flags.item()),
                k_cache=to_numpy(d["k_cache"], np.uint16), v_cache=to_numpy(d["v_cache"], np.uint16))


@pytest.mark.parametrize("name,over,sample", [
    ("tiny", {}, None),
    ("tiny", dict(N=40, B=5, Hq=8, Hkv=2, D=128, L=(10, 400), V=5000, tree="random", seed=1), None),
    ("llama8b", {}, None),
    ("llama70b", {}, ([2, 6], [1, 5])),
    # the batch sweep at its largest batch, tree and chain
    ("sweep_tree16", dict(B=128), ([0, 63, 127], [0, 5])),
    ("sweep_chain6", dict(B=128, accept=0.9), ([1, 126], [7])),
])
def test_step_matches_oracle(name, over, sample):
    say(f"step: {name} {over}")
    w = make_workload(name, **over)
    dev = device()
    g = _step(w, upload(w, dev), dev)
    batches, heads = sample if sample else (None, None)
    ref = oracle.verify_step_ref(w, batches=batches, kv_heads=heads)
    assert g["flags"] == 0
    np.testing.assert_array_equal(g["mask"], ref.mask)
    np.testing.assert_array_equal(g["depth"], ref.depth)
    sel = ~np.isnan(ref.attn_out)
    err = float(np.abs(g["out"][sel] - ref.attn_out[sel]).max())
    assert err <= ATTN_TOL, err
    excused, draws = compare_walk(ref.walk, g["path"], g["n_acc"], g["toks"])
    if excused == 0:
        np.testing.assert_array_equal(g["slots"], ref.commit_slots)
        np.testing.assert_array_equal(g["new_len"], ref.new_prefix_len)
        np.testing.assert_array_equal(g["k_cache"], ref.k_cache)
        np.testing.assert_array_equal(g["v_cache"], ref.v_cache)
    else:
        # An excused sequence took another (valid) path near a boundary: the
        # commit is still checked for every sequence, against the oracle's
        # commit of the paths the GPU walk took (the others equal the
        # oracle's own paths, which compare_walk asserted).
        k_ref, v_ref, s_ref, l_ref = oracle.kv_commit(
            w.k_tree, w.v_tree, g["path"], g["n_acc"], w.block_table, w.prefix_len, w.k_cache,
            w.v_cache)
        np.testing.assert_array_equal(g["slots"], s_ref)
        np.testing.assert_array_equal(g["new_len"], l_ref)
        np.testing.assert_array_equal(g["k_cache"], k_ref)
        np.testing.assert_array_equal(g["v_cache"], v_ref)
    say(f"  attention err {err:.2e}; accepted {g['n_acc'].tolist()}; excused {excused}/{draws}")


def test_step_is_deterministic_and_commit_idempotent():
    say("step: determinism")
    w = make_workload("tiny", N=64, B=4, Hq=32, Hkv=8, D=128, L=(300, 500), V=20000,
                      tree="random", seed=12)
    dev = device()
    d = upload(w, dev)
    a = _step(w, d, dev)
    b = _step(w, d, dev)          # same inputs; the second commit rewrites the same rows
    for k in a:
        if k != "flags":
            np.testing.assert_array_equal(a[k], b[k])
