"""The whole chain on the GPU against the oracle's chain: sampled expansion
of a candidate tree, the budget step, the mask, the without-replacement
walk and the commit, each stage fed by the previous one's device output.

Stage by stage the oracle runs on its own outputs. Where the oracle's chain
meets a decision that floating point can tip (two sampling keys within two
fp32 ulps, a budget cut within 1e-4, a walk draw within its 1e-6 window), the
sequence is excused from the stages after it; everything else is compared
bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from gpu_helpers import device, say
from synth.device import to_numpy
from synth.workloads import bf16_bits, build_paged_cache

pytestmark = pytest.mark.gpu


def _full_tree(widths):
    parent, rank, depth = [-1], [0], [0]
    i = 0
    while i < len(parent):
        if depth[i] < len(widths):
            for r in range(widths[depth[i]]):
                parent.append(i)
                rank.append(r)
                depth.append(depth[i] + 1)
        i += 1
    return np.array(parent, np.int32), np.array(rank)


def test_construct_verify_commit():
    say("pipeline: sampled expansion -> budget -> mask -> walk -> commit")
    rng = np.random.default_rng(77)
    B, V, widths, M, k = 6, 2048, (3, 3, 2, 2), 16, 3
    Hkv, D = 2, 64
    parent_c, rank = _full_tree(widths)
    Nc = parent_c.shape[0]
    draft = (rng.standard_normal((B, Nc, V)) * 2.5).astype(np.float32)
    target = (draft + rng.standard_normal((B, Nc, V)) * 0.8).astype(np.float32)
    dev = device()
    flags = tav.new_flags(dev)
    T, seed, offset = 1.0, 4, 2

    # 1. sampled children of every candidate row
    g_tok, g_lq, _ = tav.tree_expand_sample(torch.from_numpy(draft.reshape(B * Nc, V)).to(dev),
                                            k, T, seed, offset, dev_flags=flags)
    r_tok, r_lq, _ = oracle.expand_sample(draft.reshape(B * Nc, V), k, T, seed, offset)
    keys = oracle.gumbel_keys(draft.reshape(B * Nc, V), T, seed, offset)

    def candidates(tok, lq):
        tok = tok.reshape(B, Nc, k)
        lq = lq.reshape(B, Nc, k)
        token = np.zeros((B, Nc), np.int32)
        logq = np.zeros((B, Nc))
        token[:, 1:] = tok[:, parent_c[1:], rank[1:]]
        logq[:, 1:] = lq[:, parent_c[1:], rank[1:]]
        return token, logq

    gt, gl = candidates(to_numpy(g_tok), to_numpy(g_lq))
    rt, rl = candidates(r_tok, r_lq)
    live = np.ones(B, bool)
    for b in range(B):
        if not (gt[b] == rt[b]).all():
            rows = range(b * Nc, (b + 1) * Nc)
            top = [np.sort(keys[r])[::-1][:k + 1] for r in rows]
            assert any(((t[:-1] - t[1:]) <= 2 * np.spacing(np.abs(t[:-1]))).any() for t in top)
            live[b] = False

    # 2. the budget step, on each side's own candidates
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(dev)
    par_t = t(np.tile(parent_c, (B, 1)), np.int32)
    op, ot, src = tav.tree_select_topm(par_t, t(gt, np.int32), t(gl, np.float64), M,
                                       dev_flags=flags)
    rp, rtk, rs = oracle.select_topm(np.tile(parent_c, (B, 1)), rt, rl, M)
    op_n, src_n = to_numpy(op), to_numpy(src)
    for b in range(B):
        if not live[b]:
            continue
        score = np.zeros(Nc)
        for i in range(1, Nc):
            score[i] = score[parent_c[i]] + min(rl[b, i], 0.0)
        kept = set(rs[b].tolist())
        gap = min(score[list(kept)]) - max(score[i] for i in range(Nc) if i not in kept)
        if gap <= 1e-4:
            live[b] = False
            continue
        np.testing.assert_array_equal(src_n[b], rs[b])
        np.testing.assert_array_equal(op_n[b], rp[b])

    # 3. mask of the kept tree
    mask, depth = tav.tree_mask_build(op, dev_flags=flags)
    r_mask, r_depth = oracle.tree_mask(rp)
    for b in np.nonzero(live)[0]:
        np.testing.assert_array_equal(to_numpy(mask)[b].view(np.uint64), r_mask[b])

    # 4. the walk over the kept nodes' rows (gathered on the device)
    idx = src.long()
    tl_d = torch.gather(t(target, np.float32), 1, idx[:, :, None].expand(B, M, V)).contiguous()
    dl_d = torch.gather(t(draft, np.float32), 1, idx[:, :, None].expand(B, M, V)).contiguous()
    path, n_acc, toks = tav.spec_verify_sample_wor(tl_d, dl_d, op, ot, T, 9, 0, dev_flags=flags)
    ref = oracle.verify_walk(np.take_along_axis(target, rs[:, :, None], 1),
                             np.take_along_axis(draft, rs[:, :, None], 1), rp, rtk, T, 9, 0,
                             without_replacement=True)
    path_n, nacc_n, toks_n = to_numpy(path), to_numpy(n_acc), to_numpy(toks)
    for b in np.nonzero(live)[0]:
        same = (path_n[b] == ref.path[b]).all() and (toks_n[b] == ref.out_tokens[b]).all()
        if not same:
            assert ref.first_near[b] >= 0, f"sequence {b}: walk differs with no near draw"
            live[b] = False

    # 5. commit of the accepted path's K/V
    L = rng.integers(20, 60, B)
    kp = [bf16_bits(rng.standard_normal((int(l), Hkv, D)).astype(np.float32)) for l in L]
    vp = [bf16_bits(rng.standard_normal((int(l), Hkv, D)).astype(np.float32)) for l in L]
    k_cache, v_cache, table = build_paged_cache(rng, kp, vp, M, poison=False)
    k_tree = bf16_bits(rng.standard_normal((B, M, Hkv, D)).astype(np.float32))
    v_tree = bf16_bits(rng.standard_normal((B, M, Hkv, D)).astype(np.float32))
    kc, vc = t(k_cache.view(np.int16), np.int16), t(v_cache.view(np.int16), np.int16)
    slots, new_len = tav.kv_commit_path(
        t(k_tree.view(np.int16), np.int16), t(v_tree.view(np.int16), np.int16), path, n_acc,
        t(table, np.int32), t(L, np.int32), kc, vc, dev_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    rk, rv, rslots, rlen = oracle.kv_commit(k_tree, v_tree, ref.path, ref.n_accepted, table, L,
                                            k_cache, v_cache)
    slots_n, len_n = to_numpy(slots), to_numpy(new_len)
    for b in np.nonzero(live)[0]:
        np.testing.assert_array_equal(slots_n[b], rslots[b])
        assert len_n[b] == rlen[b]
    if live.all():
        np.testing.assert_array_equal(to_numpy(kc).view(np.uint16), rk)
        np.testing.assert_array_equal(to_numpy(vc).view(np.uint16), rv)
    say(f"  sequences compared through every stage: {int(live.sum())} of {B}")
    assert live.sum() >= B - 1
