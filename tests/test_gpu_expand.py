"""GPU tree expansion (top-k draft tokens, log q, entropy) against the oracle.

Tokens are compared bit for bit (the ranking compares the fp32 logits). log q
and the entropy use fp32 exponentials summed in fp64: each term is within
about 1e-7 relative and y = (x - M)/T is rounded once in fp32, so both are
within about 1e-6 of the fp64 oracle; the bound asserted is EXPAND_TOL."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from synth.device import to_numpy

from gpu_helpers import device, say

pytestmark = pytest.mark.gpu
EXPAND_TOL = 1e-5


def run_expand(x, k, T, dev):
    flags = tav.new_flags(dev)
    tok, lq, ent = tav.tree_expand_topk(torch.from_numpy(np.ascontiguousarray(x)).to(dev), k, T,
                                        dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(tok), to_numpy(lq), to_numpy(ent), int(flags.item())


@pytest.mark.parametrize("R,V,k,T,scale", [
    (64, 128256, 4, 1.0, 3.0),
    (16, 128256, 16, 0.7, 3.0),
    (8, 151936, 8, 1.3, 1.0),
    (33, 1000, 5, 1.0, 2.0),
    (7, 777, 3, 1.0, 2.0),
    (9, 4097, 16, 1.0, 0.5),
    (5, 8, 8, 1.0, 1.0),
])
def test_expand_matches_oracle(R, V, k, T, scale):
    say(f"expand: R={R} V={V} k={k} T={T}")
    rng = np.random.default_rng(V + k)
    x = (rng.standard_normal((R, V)) * scale).astype(np.float32)
    tok, lq, ent, flags = run_expand(x, k, T, device())
    assert flags == 0
    rt, rl, re = oracle.expand_topk(x, k, T)
    np.testing.assert_array_equal(tok, rt)
    e1, e2 = float(np.abs(lq - rl).max()), float(np.abs(ent - re).max())
    say(f"  max |dlogq| {e1:.2e}, max |dH| {e2:.2e}")
    assert e1 <= EXPAND_TOL and e2 <= EXPAND_TOL


def test_expand_ties_signed_zero_and_neg_inf():
    say("expand: ties across workgroups, -0/+0, -inf entries")
    V, k = 20000, 6
    x = np.full((4, V), -3.0, np.float32)
    x[0, [4095, 4096, 9000, 12]] = 2.0          # ties across a workgroup boundary
    x[1, 5:V:7] = 1.0                            # thousands of equal maxima
    x[2, 9] = 0.0
    x[2, 3] = -0.0
    x[2, 100:] = -np.inf                         # most of the row has q = 0
    x[3, :] = -np.inf
    x[3, [7, 19999]] = 0.5
    tok, lq, ent, flags = run_expand(x, k, 1.0, device())
    assert flags == 0
    rt, rl, re = oracle.expand_topk(x, k, 1.0)
    np.testing.assert_array_equal(tok, rt)
    fin = np.isfinite(rl)
    np.testing.assert_array_equal(np.isfinite(lq), fin)
    assert float(np.abs(lq[fin] - rl[fin]).max()) <= EXPAND_TOL
    assert float(np.abs(ent - re).max()) <= EXPAND_TOL
    assert tok[0, :3].tolist() == [12, 4095, 4096]


def test_expand_flags_non_finite_rows():
    say("expand: NaN and all -inf rows flagged")
    x = np.random.default_rng(1).standard_normal((3, 5000)).astype(np.float32)
    x[1, 77] = np.nan
    x[2, :] = -np.inf
    tok, lq, ent, flags = run_expand(x, 4, 1.0, device())
    assert flags & tav.FLAG_NONFINITE_LOGITS
    assert (tok[1:] == -1).all() and np.isnan(ent[1:]).all()
    rt, rl, re = oracle.expand_topk(x[:1], 4, 1.0)
    np.testing.assert_array_equal(tok[:1], rt)


def test_topk_large_logits_match_oracle():
    """Blocks of equal large logits at T != 1: the sums rebase every term to
    the wave's maximum with products rounded on their own, so the maximum's
    term is exactly 1 (a fused product would leave its rounding error there
    and bend log q by it)."""
    say("expand topk: large equal logits, T = 0.9")
    rng = np.random.default_rng(41)
    dev = device()
    for big in (1e30, 1e10, 1e4, 100.0):
        x = rng.standard_normal((3, 9000)).astype(np.float32)
        x[0, 100:400] = big
        x[1, 5000:5100] = big
        x[2, ::7] = big
        flags = tav.new_flags(dev)
        tok, lq, ent = tav.tree_expand_topk(torch.from_numpy(x).to(dev), 6, 0.9, dev_flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        rt, rl, re = oracle.expand_topk(x, 6, 0.9)
        np.testing.assert_array_equal(to_numpy(tok), rt)
        np.testing.assert_allclose(to_numpy(lq), rl, rtol=0, atol=1e-5)
        np.testing.assert_allclose(to_numpy(ent), re, rtol=0, atol=1e-5)
