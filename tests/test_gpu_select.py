"""GPU parity: tree_select_topm (budget-constrained top-M subtree) and
tree_widths_by_entropy (entropy-ranked branching) against the oracle, bit
for bit, and the construction pipeline tree_expand_topk -> tree_select_topm
(and -> widths) against the oracle's."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import device, say
from synth import random_parent
from synth.device import to_numpy

pytestmark = pytest.mark.gpu


def _run(parent, token, logq, M):
    dev = device()
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(dev)
    flags = tav.new_flags(dev)
    op, ot, src = tav.tree_select_topm(t(parent, np.int32), t(token, np.int32),
                                       t(logq, np.float64), M, dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(op), to_numpy(ot), to_numpy(src), int(flags.item())


def _scores(rng, B, Nc):
    lq = -np.round(rng.exponential(1.0, (B, Nc)) * 8) / 8    # coarse: many equal scores
    lq[rng.random((B, Nc)) < 0.05] = -np.inf
    lq[rng.random((B, Nc)) < 0.03] = 3e-17                     # rounding above 0
    fine = rng.random((B, Nc)) < 0.5
    lq[fine] = np.log(rng.uniform(1e-6, 1.0, int(fine.sum())))
    return lq


@pytest.mark.parametrize("B,Nc,M", [
    (3, 1, 1), (4, 2, 1), (4, 2, 2), (8, 63, 17), (8, 64, 64), (8, 65, 40), (16, 300, 64),
    (4, 357, 64), (2, 1024, 256), (2, 1024, 1), (2, 1024, 1024), (64, 40, 12),
])
def test_matches_oracle(B, Nc, M):
    say(f"select: B={B} Nc={Nc} M={M}")
    rng = np.random.default_rng(Nc * 1000 + M)
    parent = np.stack([random_parent(rng, Nc) for _ in range(B)])
    token = rng.integers(0, 128256, (B, Nc))
    logq = _scores(rng, B, Nc)
    op, ot, src, flags = _run(parent, token, logq, M)
    assert flags == 0
    rp, rt, rs = oracle.select_topm(parent, token, logq, M)
    np.testing.assert_array_equal(src, rs)
    np.testing.assert_array_equal(op, rp)
    np.testing.assert_array_equal(ot, rt)


def test_deep_chain_and_star():
    say("select: chain of 1024, star of 1024")
    rng = np.random.default_rng(5)
    Nc = 1024
    chain = np.arange(-1, Nc - 1)[None]
    star = np.r_[-1, np.zeros(Nc - 1, int)][None]
    for parent in (chain, star):
        logq = np.log(rng.uniform(0.5, 1.0, (1, Nc)))
        token = rng.integers(0, 1000, (1, Nc))
        for M in (1, 100, 1024):
            op, ot, src, flags = _run(parent, token, logq, M)
            assert flags == 0
            rp, rt, rs = oracle.select_topm(parent, token, logq, M)
            np.testing.assert_array_equal(src, rs)
            np.testing.assert_array_equal(op, rp)


def test_flags_for_bad_inputs():
    say("select: flags")
    parent = np.array([[-1, 0, 0, 1], [-1, 0, 3, 1]])
    logq = np.zeros((2, 4))
    *_, flags = _run(parent, parent, logq, 2)
    assert flags == 0x1          # TAV_FLAG_BAD_PARENT
    logq[0, 2] = np.nan
    *_, flags = _run(parent[:1], parent[:1], logq[:1], 2)
    assert flags == 0x4          # TAV_FLAG_NONFINITE_LOGITS


def _full_tree(widths):
    """Level-order candidate tree where every node of depth d has widths[d]
    children; returns parent and each node's rank among its siblings."""
    parent, rank, depth = [-1], [0], [0]
    i = 0
    while i < len(parent):
        if depth[i] < len(widths):
            for r in range(widths[depth[i]]):
                parent.append(i)
                rank.append(r)
                depth.append(depth[i] + 1)
        i += 1
    return np.array(parent), np.array(rank)


def test_expand_then_select_pipeline():
    """Expansion and budget step on the GPU against the oracle's, on a
    Llama-3-8B-shaped candidate tree (widths 4, 4, 3, 2, 2: 357 nodes, 64
    kept) with a 4096-token vocabulary."""
    say("select: expand -> select pipeline")
    rng = np.random.default_rng(21)
    B, V, widths, M = 6, 4096, (4, 4, 3, 2, 2), 64
    parent, rank = _full_tree(widths)
    Nc = parent.shape[0]
    k = max(widths)
    rows = (rng.standard_normal((B * Nc, V)) * 3).astype(np.float32)

    dev = device()
    flags = tav.new_flags(dev)
    top_tok, top_lq, _ = tav.tree_expand_topk(torch.from_numpy(rows).to(dev), k, 1.0,
                                              dev_flags=flags)
    g_tok = to_numpy(top_tok).reshape(B, Nc, k)
    g_lq = to_numpy(top_lq).reshape(B, Nc, k)
    r_tok, r_lq, _ = oracle.expand_topk(rows, k, 1.0)
    r_tok = r_tok.reshape(B, Nc, k)
    r_lq = r_lq.reshape(B, Nc, k)

    def candidates(tok, lq):
        token = np.zeros((B, Nc), np.int64)
        logq = np.zeros((B, Nc))
        token[:, 1:] = tok[:, parent[1:], rank[1:]]
        logq[:, 1:] = lq[:, parent[1:], rank[1:]]
        return token, logq

    gt, gl = candidates(g_tok, g_lq)
    rt, rl = candidates(r_tok, r_lq)
    np.testing.assert_array_equal(gt, rt)
    op, ot, src, f2 = _run(np.tile(parent, (B, 1)), gt, gl, M)
    assert int(flags.item()) == 0 and f2 == 0
    rp, rtk, rs = oracle.select_topm(np.tile(parent, (B, 1)), rt, rl, M)
    # the two sides' log q agree to about 1e-6, so a sequence may differ only
    # if the oracle's cut (last kept against best dropped) is that close
    for b in range(B):
        score = np.zeros(Nc)
        for i in range(1, Nc):
            score[i] = score[parent[i]] + min(rl[b, i], 0.0)
        kept = set(rs[b].tolist())
        gap = min(score[list(kept)]) - max(score[i] for i in range(Nc) if i not in kept)
        if gap > 1e-4:
            np.testing.assert_array_equal(src[b], rs[b])
            np.testing.assert_array_equal(op[b], rp[b])
            np.testing.assert_array_equal(ot[b], rtk[b])


# ---- entropy-ranked widths ---------------------------------------------------

def _widths(h, lo, hi):
    dev = device()
    flags = tav.new_flags(dev)
    w = tav.tree_widths_by_entropy(torch.from_numpy(np.ascontiguousarray(h)).to(dev), lo, hi,
                                   dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(w), int(flags.item())


@pytest.mark.parametrize("B,F,lo,hi", [
    (4, 1, 1, 4), (8, 7, 1, 4), (8, 64, 1, 4), (4, 65, 2, 5), (16, 200, 1, 4), (3, 513, 0, 7),
    (2, 1024, 1, 4), (64, 16, 1, 1),
])
def test_widths_match_oracle(B, F, lo, hi):
    say(f"widths: B={B} F={F} w={lo}..{hi}")
    rng = np.random.default_rng(F * 10 + lo)
    h = np.round(rng.exponential(2.0, (B, F)) * 4) / 4     # coarse: many equal entropies
    h[rng.random((B, F)) < 0.05] = np.inf
    w, flags = _widths(h, lo, hi)
    assert flags == 0
    np.testing.assert_array_equal(w, oracle.widths_by_entropy(h, lo, hi))


def test_widths_from_expansion_entropy():
    """Entropies from tree_expand_topk on the GPU against the oracle's
    expand_topk, ranked on both sides; a row may differ only where two
    entropies are within the expansion's tolerance of each other."""
    say("widths: from expansion entropies")
    rng = np.random.default_rng(31)
    B, F, V = 8, 24, 4096
    rows = (rng.standard_normal((B * F, V)) * rng.uniform(0.5, 4, (B * F, 1))).astype(np.float32)
    dev = device()
    _, _, ent = tav.tree_expand_topk(torch.from_numpy(rows).to(dev), 4, 1.0)
    w, flags = _widths(to_numpy(ent).reshape(B, F), 1, 4)
    assert flags == 0
    _, _, r_ent = oracle.expand_topk(rows, 4, 1.0)
    r_ent = r_ent.reshape(B, F)
    ref = oracle.widths_by_entropy(r_ent, 1, 4)
    compared = 0
    for b in range(B):
        gaps = np.diff(np.sort(r_ent[b]))
        if gaps.min() > 1e-4:
            np.testing.assert_array_equal(w[b], ref[b])
            compared += 1
    assert compared == B   # these inputs leave every row's entropies well apart


def test_widths_flag_nan():
    h = np.zeros((1, 5))
    h[0, 3] = np.nan
    _, flags = _widths(h, 1, 4)
    assert flags == 0x4
