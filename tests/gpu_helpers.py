"""Helpers for the GPU parity tests: run the library, compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from synth.device import to_numpy, upload

ATTN_TOL = 2e-3     # max abs error of attention outputs vs the fp64 oracle
P_TOL = 1e-5        # max abs error of target probabilities
EXCUSE_RATE = 1e-4  # excused walk mismatches per draw


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def run_mask(w, dev):
    d = upload(w, dev, logits=False)
    flags = tav.new_flags(dev)
    mask, depth = tav.tree_mask_build(d["parent"], dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(mask, np.uint64), to_numpy(depth), int(flags.item())


def run_attention(w, dev, mask=None, max_prefix_len=None):
    d = upload(w, dev, logits=False)
    flags = tav.new_flags(dev)
    if mask is None:
        mask, _ = tav.tree_mask_build(d["parent"], dev_flags=flags)
    else:
        mask = torch.from_numpy(mask.view(np.int64)).to(dev)
    out = tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"],
                               d["block_table"], d["prefix_len"],
                               w.max_prefix_len if max_prefix_len is None else max_prefix_len,
                               mask, scale=w.scale, dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(out), int(flags.item())


def run_walk(w, dev, seed=None, offset=None, wor=False):
    d = upload(w, dev)
    flags = tav.new_flags(dev)
    fn = tav.spec_verify_sample_wor if wor else tav.spec_verify_sample
    path, n_acc, toks = fn(
        d["target_logits"], d["draft_logits"], d["parent"], d["token"], w.temperature,
        w.philox_seed if seed is None else seed, w.philox_offset if offset is None else offset,
        dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(path), to_numpy(n_acc), to_numpy(toks), int(flags.item())


def walk_arrays(tl, dl, parent, token, T, seed, offset, dev, wor=False):
    """Run the device walk on raw numpy arrays (``wor``: the without-replacement
    sibling rule)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    flags = tav.new_flags(dev)
    fn = tav.spec_verify_sample_wor if wor else tav.spec_verify_sample
    path, n_acc, toks = fn(t(tl), t(dl), t(parent.astype(np.int32)), t(token.astype(np.int32)),
                           T, seed, offset, dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(path), to_numpy(n_acc), to_numpy(toks), int(flags.item())


def compare_walk(ref: "oracle.WalkResult", path, n_acc, toks):
    """Bit-exact comparison with the boundary rule.

    A sequence may differ from the oracle only if the oracle met a draw within
    1e-6 of its decision boundary, and only after the path prefix accepted
    before that draw. Returns (excused sequences, total draws); asserts the
    excused count stays under 1e-4 of the draws.
    """
    B = path.shape[0]
    excused = 0
    for b in range(B):
        same = (n_acc[b] == ref.n_accepted[b] and (path[b] == ref.path[b]).all()
                and (toks[b] == ref.out_tokens[b]).all())
        if same:
            continue
        fn = int(ref.first_near[b])
        assert fn >= 0, (f"sequence {b} differs with no near-boundary draw: gpu path "
                         f"{path[b][:8]} acc {n_acc[b]} tokens {toks[b][:8]}; oracle path "
                         f"{ref.path[b][:8]} acc {ref.n_accepted[b]} tokens {ref.out_tokens[b][:8]}")
        assert (path[b, :fn + 1] == ref.path[b, :fn + 1]).all(), f"sequence {b} differs early"
        excused += 1
    draws = int(ref.draws.sum())
    assert excused <= EXCUSE_RATE * draws, (excused, draws)
    return excused, draws
