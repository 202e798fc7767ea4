"""GPU parity: tree_attn_verify against the fp64 oracle on the same bf16 inputs.

Small cases span several 64-key tiles, ragged prefix tails, split-K, several
row blocks and several 64-node tree tiles; full-size cases compare a sample of
(sequence, KV head) pairs the oracle computes in seconds.
"""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import ATTN_TOL, device, run_attention, say
from synth import make_workload
from synth.device import to_numpy, upload

pytestmark = pytest.mark.gpu

CASES = [
    dict(N=5, B=1, Hq=1, Hkv=1, D=64, L=(128, 128), tree="example"),
    dict(N=7, B=2, Hq=4, Hkv=2, D=64, L=(37, 300), tree="chain"),
    dict(N=40, B=3, Hq=8, Hkv=2, D=128, L=(1, 250), tree="random"),
    dict(N=1, B=2, Hq=8, Hkv=8, D=128, L=(64, 65), tree="chain"),
    dict(N=9, B=2, Hq=4, Hkv=1, D=128, L=(0, 0), tree="random"),
    dict(N=64, B=2, Hq=64, Hkv=8, D=128, L=(500, 700), tree="random"),     # 512 rows: 2 row blocks
    dict(N=130, B=1, Hq=8, Hkv=4, D=64, L=(70, 70), tree="random"),        # 3 tree tiles
    dict(N=256, B=1, Hq=2, Hkv=1, D=128, L=(3000, 3000), tree="random"),   # 4 tree tiles, split-K
    dict(N=16, B=4, Hq=32, Hkv=8, D=128, L=(2047, 2049), tree="random"),
    dict(N=6, B=3, Hq=32, Hkv=8, D=128, L=(2048, 2048), tree="chain"),
    dict(N=20, B=2, Hq=8, Hkv=2, D=128, L=(1000, 1100), tree="random"),    # 80 rows: 4 waves x 32
    dict(N=48, B=1, Hq=64, Hkv=8, D=64, L=(513, 700), tree="random"),      # 384 rows, D=64, 2 row blocks
    # the small trees of the tree-size sweep at 70B-shaped heads (8 to 32 rows)
    dict(N=1, B=2, Hq=64, Hkv=8, D=128, L=(700, 900), tree="chain"),
    dict(N=2, B=2, Hq=64, Hkv=8, D=128, L=(700, 900), tree="chain"),
    dict(N=4, B=2, Hq=64, Hkv=8, D=128, L=(300, 1500), tree="random"),
    # 129..256 rows at batch one, which eight row waves cannot spread over
    # the device: four row waves in two key sets, two row blocks (the
    # second ragged), 16 splits
    dict(N=40, B=1, Hq=32, Hkv=8, D=64, L=(2000, 2000), tree="random"),
    dict(N=60, B=1, Hq=32, Hkv=8, D=128, L=(2600, 2600), tree="random"),
]


def _check(w, out, flags, batches=None, kv_heads=None):
    mask, _ = oracle.tree_mask(w.parent)
    ref = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache, w.block_table,
                                w.prefix_len, mask, scale=w.scale, batches=batches,
                                kv_heads=kv_heads)
    assert flags == 0
    sel = ~np.isnan(ref)
    assert sel.any()
    err = float(np.abs(out[sel] - ref[sel]).max())
    assert np.isfinite(out).all()
    assert err <= ATTN_TOL, err
    return err


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: f"N{c['N']}-G{c['Hq']//c['Hkv']}-D{c['D']}-L{c['L'][1]}")
def test_attention_matches_oracle(cfg):
    say(f"attention: {cfg}")
    w = make_workload("tiny", with_logits=False, seed=cfg["N"] + cfg["L"][1], **cfg)
    out, flags = run_attention(w, device())
    err = _check(w, out, flags)
    say(f"  max abs err {err:.2e}")


# Prefix lengths far apart within one batch under a split plan: splits of
# one sequence range from many tiles to none (a sequence with fewer tiles
# than splits leaves some empty), and the partials of long and short
# sequences are merged side by side.
SPLIT_CASES = [
    # (B, N, Hq, Hkv, D, max prefix, prefix lengths)
    (5, 9, 8, 2, 128, 3000, [0, 3000, 5, 64, 2000]),
    (6, 16, 64, 8, 128, 3000, [3000, 0, 0, 0, 10, 3000]),
    (4, 7, 8, 2, 64, 4096, [0, 0, 1, 0]),                 # more ranges than tiles
    (3, 70, 8, 4, 128, 5000, [4999, 63, 1500]),           # two tree tiles
    (8, 64, 64, 8, 128, 2000, [2000, 1, 640, 1999, 65, 700, 1300, 128]),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"B{c[0]}-N{c[1]}-D{c[4]}")
def test_attention_splits_with_prefix_lengths_far_apart(case):
    B, N, Hq, Hkv, D, Lmax, lens = case
    plan = tav.attn_plan(B, N, Hq, Hkv, D, Lmax, torch.cuda.get_device_properties(0).multi_processor_count, 1)
    say(f"attention, split ranges: {case} plan {plan}")
    assert plan["splits"] >= 2
    w = make_workload("tiny", with_logits=False, seed=B * 100 + N, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D,
                      L=(Lmax, Lmax), tree="random")
    # shorter prefixes than the cache holds: the slots past them must not count
    w.prefix_len[:] = lens
    out, flags = run_attention(w, device(), max_prefix_len=Lmax)
    err = _check(w, out, flags)
    say(f"  max abs err {err:.2e}")


def test_attention_70b_full_size_sampled():
    say("attention: llama70b full size, sampled heads")
    w = make_workload("llama70b", with_logits=False)
    out, flags = run_attention(w, device())
    err = _check(w, out, flags, batches=[0, 5, 7], kv_heads=[0, 3, 7])
    say(f"  max abs err {err:.2e}")


def test_attention_70b_tp8_share_sampled():
    say("attention: one GPU's share of the 70B-shaped layer under 8-way tensor parallelism")
    w = make_workload("llama70b_tp8", with_logits=False)
    out, flags = run_attention(w, device())
    err = _check(w, out, flags, batches=[0, 3, 6])
    say(f"  max abs err {err:.2e}")


def test_attention_long_context_sampled():
    say("attention: long context, sampled heads")
    w = make_workload("long", with_logits=False)
    out, flags = run_attention(w, device())
    err = _check(w, out, flags, batches=[1], kv_heads=[2, 6])
    say(f"  max abs err {err:.2e}")


def test_attention_8b_full():
    say("attention: llama8b full")
    w = make_workload("llama8b", with_logits=False)
    out, flags = run_attention(w, device())
    err = _check(w, out, flags)
    say(f"  max abs err {err:.2e}")


def test_attention_is_deterministic():
    say("attention: determinism")
    w = make_workload("tiny", N=64, B=2, Hq=64, Hkv=8, D=128, L=(900, 1000), tree="random",
                      with_logits=False, seed=4)
    a, _ = run_attention(w, device())
    b, _ = run_attention(w, device())
    np.testing.assert_array_equal(a, b)


def test_attention_flags_bad_block_and_capacity():
    say("attention: bad block flag")
    w = make_workload("tiny", N=5, B=2, L=(100, 100), with_logits=False, seed=2)
    w.block_table[1, 2] = w.k_cache.shape[0] + 5        # outside the cache
    out, flags = run_attention(w, device())
    assert flags & tav.FLAG_BAD_BLOCK
    # sequence 0 is unaffected
    mask, _ = oracle.tree_mask(w.parent)
    w.block_table[1, 2] = 0
    ref = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache, w.block_table,
                                w.prefix_len, mask, scale=w.scale, batches=[0])
    assert np.abs(out[0] - ref[0]).max() <= ATTN_TOL
    say("attention: capacity flag")
    w2 = make_workload("tiny", N=5, B=1, L=(100, 100), with_logits=False, seed=2)
    dev = device()
    d = upload(w2, dev, logits=False)
    flags_t = tav.new_flags(dev)
    mask_t, _ = tav.tree_mask_build(d["parent"])
    tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                         d["block_table"], d["prefix_len"], 64, mask_t, dev_flags=flags_t)
    torch.cuda.synchronize()
    assert int(flags_t.item()) & tav.FLAG_CAPACITY
