"""GPU greedy verification (temperature 0) against the oracle, bit for bit.

The decisions are comparisons of fp32 logits, so the device and the oracle
take them on the same values and must agree exactly (ties go to the lowest
token id on both sides)."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from synth import make_workload
from synth.device import to_numpy

from gpu_helpers import device, say

pytestmark = pytest.mark.gpu


def greedy_arrays(tl, parent, token, dev, draft=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    flags = tav.new_flags(dev)
    path, n_acc, toks = tav.spec_verify_sample(
        t(tl), None if draft is None else t(draft), t(parent.astype(np.int32)),
        t(token.astype(np.int32)), 0.0, 0, 0, dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(path), to_numpy(n_acc), to_numpy(toks), int(flags.item())


def check(tl, parent, token, dev, draft=None):
    path, n_acc, toks, flags = greedy_arrays(tl, parent, token, dev, draft)
    assert flags == 0, hex(flags)
    ref = oracle.verify_greedy(tl, parent, token)
    np.testing.assert_array_equal(n_acc, ref.n_accepted)
    np.testing.assert_array_equal(path, ref.path)
    np.testing.assert_array_equal(toks, ref.out_tokens)
    return n_acc


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", dict(N=40, B=64, V=1000, tree="random", seed=5)),
    ("tiny", dict(N=256, B=4, V=3000, tree="random", seed=6)),
    ("tiny", dict(N=1, B=50, V=5000, tree="chain", seed=7)),
    ("tiny", dict(N=30, B=16, V=777, tree="random", seed=9)),
    ("tiny", dict(N=12, B=32, V=4097, tree="chain", seed=8, sigma_d=0.1)),
    ("llama8b", {}),
    ("llama70b", {}),
    ("long", {}),
    ("sweep_tree16", dict(B=128, accept=0.9)),
])
def test_greedy_matches_oracle(name, over):
    say(f"greedy: {name} {over}")
    w = make_workload(name, **over)
    dev = device()
    n_acc = check(w.target_logits, w.parent, w.token, dev, draft=w.draft_logits)
    say(f"  accepted {n_acc.tolist()[:8]}")


@pytest.mark.parametrize("N,V", [(8, 1000), (64, 128256), (200, 4097)])
def test_greedy_long_accepted_chains(N, V):
    # node i carries the target's choice at node i-1 except where a mismatch
    # is planted, so the walk runs long and stops at a known place
    say(f"greedy: matching chains N={N} V={V}")
    rng = np.random.default_rng(N)
    B = 6
    tl = (rng.standard_normal((B, N, V)) * 3).astype(np.float32)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    token = np.zeros((B, N), np.int32)
    token[:, 1:] = tl[:, :-1].argmax(axis=2)
    for b in range(1, B):
        k = int(rng.integers(1, N)) if N > 1 else 0
        token[b, k] = (token[b, k] + 1) % V
    n_acc = check(tl, parent, token, device())
    assert n_acc[0] == N - 1


def test_greedy_ties_and_signed_zero_take_the_lowest_token():
    say("greedy: ties across workgroup chunks")
    V, N, B = 20000, 2, 4
    tl = np.full((B, N, V), -5.0, np.float32)
    tl[0, 0, [4095, 4096, 9000]] = 2.0          # across the first chunk boundary
    tl[1, 0, [12000, 100, 19999]] = 1.5
    tl[2, 0, 9] = 0.0
    tl[2, 0, 3] = -0.0                          # -0 and +0 are equal: token 3
    tl[3, 0, V - 1] = 7.0                       # the last token alone
    tl[:, 1, 0] = 1.0
    parent = np.tile(np.array([-1, 0], np.int32), (B, 1))
    token = np.array([[0, 4096], [0, 100], [0, 3], [0, 5]], np.int32)
    check(tl, parent, token, device())
    ref = oracle.verify_greedy(tl, parent, token)
    assert ref.out_tokens[0, 0] == 4095 and ref.n_accepted[0] == 0
    assert ref.n_accepted[1] == 1 and ref.n_accepted[2] == 1


def test_greedy_flags_non_finite_rows():
    say("greedy: NaN, -inf row and +inf flagged")
    dev = device()
    V = 5000
    parent = np.array([[-1, 0, 0]], np.int32)
    token = np.array([[0, 1, 2]], np.int32)
    for poison in ("nan", "neg_inf_row", "pos_inf"):
        tl = np.random.default_rng(1).standard_normal((1, 3, V)).astype(np.float32)
        if poison == "nan":
            tl[0, 0, 4321] = np.nan
        elif poison == "neg_inf_row":
            tl[0, 0, :] = -np.inf
        else:
            tl[0, 0, 17] = np.inf
        _, n_acc, toks, flags = greedy_arrays(tl, parent, token, dev)
        assert flags & tav.FLAG_NONFINITE_LOGITS, poison
        assert n_acc[0] == 0 and (toks[0] == -1).all()


def test_greedy_is_deterministic_and_leaves_the_workspace_zero():
    say("greedy: determinism, workspace left zero")
    dev = device()
    w = make_workload("tiny", N=40, B=64, V=20000, tree="random", seed=3)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ws = tav.new_sampler_workspace(w.B, w.N, w.V, dev)
    outs = []
    for _ in range(3):
        flags = tav.new_flags(dev)
        r = tav.spec_verify_sample(t(w.target_logits), None, t(w.parent), t(w.token), 0.0, 0, 0,
                                   workspace=ws, dev_flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        outs.append([to_numpy(x) for x in r])
        assert int(ws.count_nonzero().item()) == 0
    for o in outs[1:]:
        for x, y in zip(outs[0], o):
            np.testing.assert_array_equal(x, y)
