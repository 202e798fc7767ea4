"""GPU sampled expansion (k draft tokens drawn without replacement by
Gumbel top-k) against the oracle, and the sampled tree verified by the
without-replacement walk on the GPU.

Both sides form every key the same way in float64 (x/T + G, G = -log(-log u)
on the same 53-bit uniform); they differ only in their log routines, each
within an ulp, so two keys can be ordered differently only if they agree to
about 1e-15 relative. A row may therefore differ from the oracle only if two
of its k + 1 best oracle keys are within 1e-12 relative of each other, and
such rows must be under 1e-4 of all rows (none at these sizes). log q and the
entropy are as for tree_expand_topk.
"""

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import tree_attention_verification_ancestor_amd as tav
from synth.device import to_numpy

from gpu_helpers import compare_walk, device, say, walk_arrays

pytestmark = pytest.mark.gpu
EXPAND_TOL = 1e-5
TIE_REL = 1e-12          # keys closer than this may be ordered either way
EXCUSE_RATE = 1e-4       # rows


def run_sample(x, k, T, seed, offset):
    dev = device()
    flags = tav.new_flags(dev)
    tok, lq, ent = tav.tree_expand_sample(torch.from_numpy(np.ascontiguousarray(x)).to(dev), k, T,
                                          seed, offset, dev_flags=flags)
    torch.cuda.synchronize()
    return to_numpy(tok), to_numpy(lq), to_numpy(ent), int(flags.item())


def _near_tie(keys_row, k):
    top = np.sort(keys_row)[::-1][:k + 1]
    top = top[np.isfinite(top)]
    gaps = top[:-1] - top[1:]
    return bool((gaps <= TIE_REL * np.abs(top[:-1])).any())


def _compare(x, k, T, seed, offset):
    tok, lq, ent, flags = run_sample(x, k, T, seed, offset)
    assert flags == 0
    rt, rl, re = oracle.expand_sample(x, k, T, seed, offset)
    keys = oracle.gumbel_keys(x, T, seed, offset)
    R = x.shape[0]
    excused = 0
    for r in range(R):
        if (tok[r] == rt[r]).all():
            ok = np.isfinite(rl[r])
            np.testing.assert_allclose(lq[r][ok], rl[r][ok], rtol=0, atol=EXPAND_TOL)
            assert (lq[r][~ok] == rl[r][~ok]).all()
            continue
        assert _near_tie(keys[r], k), f"row {r}: gpu {tok[r]} oracle {rt[r]}"
        excused += 1
    assert excused <= EXCUSE_RATE * R, (excused, R)
    assert float(np.abs(ent - re).max()) <= EXPAND_TOL
    return tok


@pytest.mark.parametrize("R,V,k,T,scale,seed,offset", [
    (64, 128256, 4, 1.0, 3.0, 1, 0),
    (16, 128256, 16, 0.7, 3.0, 2, 5),
    (8, 151936, 8, 1.3, 1.0, 3, 9),
    (33, 1000, 5, 1.0, 2.0, 4, 1),
    (9, 4097, 16, 1.0, 0.5, 5, 2),
    (5, 8, 8, 1.0, 1.0, 6, 3),
    (7, 2049, 3, 1.0, 12.0, 7, 4),
])
def test_sample_matches_oracle(R, V, k, T, scale, seed, offset):
    say(f"expand sample: R={R} V={V} k={k} T={T} scale={scale}")
    rng = np.random.default_rng(V + 7 * k)
    x = (rng.standard_normal((R, V)) * scale).astype(np.float32)
    tok = _compare(x, k, T, seed, offset)
    for r in range(R):
        assert len(set(tok[r].tolist())) == k


def test_sample_edge_rows_match_oracle():
    """Rows that take the rarer paths: a block of equal huge logits (every
    key ties in float64, so the wave resolves its many contenders exactly
    and the lowest tokens win), rows masked to -inf except a few tokens
    (fewer finite tokens than k: the lowest -inf tokens follow), a whole
    masked share, and a row of equal logits."""
    say("expand sample: edge rows")
    rng = np.random.default_rng(31)
    R, V, k = 6, 9000, 6
    x = rng.standard_normal((R, V)).astype(np.float32)
    x[0, 100:400] = 1e30
    x[1, :] = -np.inf
    x[1, [7, 4100, 8999]] = (0.5, 2.0, -1.0)
    x[2, 2048:6144] = -np.inf
    x[3, :] = 0.25
    x[4, :] = -np.inf
    x[4, 3] = 1.0
    x[5, 5000:5100] = 40.0
    tok = _compare(x, k, 0.9, 17, 2)
    assert (tok[0] == np.arange(100, 100 + k)).all()
    assert sorted(tok[1][:3].tolist()) == [7, 4100, 8999]   # the finite ones first
    assert tok[1][3:].tolist() == [0, 1, 2]                 # then the lowest -inf tokens


def test_one_draw_follows_q_on_gpu():
    say("expand sample: chi-square of single draws, 2e5 rows")
    rng = np.random.default_rng(8)
    V, R = 8, 200000
    row = (rng.standard_normal(V) * 1.2).astype(np.float32)
    tok, _, _, flags = run_sample(np.tile(row, (R, 1)), 1, 1.0, 11, 0)
    assert flags == 0
    q = scipy.special.softmax(row.astype(np.float64))
    counts = np.bincount(tok[:, 0], minlength=V)
    stat = float(((counts - q * R) ** 2 / (q * R)).sum())
    assert stat < 24.32, stat


def test_sampled_tree_is_verified_losslessly_on_gpu():
    """Root with 3 children drawn on the GPU, walked on the GPU by the
    without-replacement rule: the first emitted token follows p."""
    say("expand sample: sampled children -> spec_verify_sample_wor, 2e5 trees")
    rng = np.random.default_rng(9)
    V, R, k = 6, 200000, 3
    pl = (rng.standard_normal(V) * 1.2).astype(np.float32)
    ql = np.r_[[2.5], rng.standard_normal(V - 1)].astype(np.float32)
    tok, _, _, flags = run_sample(np.tile(ql, (R, 1)), k, 1.0, 12, 0)
    assert flags == 0
    tl = np.broadcast_to(pl, (R, k + 1, V)).copy()
    dl = np.broadcast_to(ql, (R, k + 1, V)).copy()
    parent = np.tile(np.array([-1] + [0] * k, np.int32), (R, 1))
    token = np.zeros((R, k + 1), np.int32)
    token[:, 1:] = tok
    path, n_acc, toks, f2 = walk_arrays(tl, dl, parent, token, 1.0, 13, 0, device(), wor=True)
    assert f2 == 0
    p = scipy.special.softmax(pl.astype(np.float64))
    counts = np.bincount(toks[:, 0], minlength=V)
    stat = float(((counts - p * R) ** 2 / (p * R)).sum())
    assert stat < 20.52, stat
    ref = oracle.verify_walk(tl, dl, parent, token, 1.0, 13, 0, without_replacement=True)
    compare_walk(ref, path, n_acc, toks)


def test_sample_is_deterministic_and_top_k_unchanged():
    say("expand sample: determinism; top-k path unchanged")
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((12, 20000)) * 2).astype(np.float32)
    a = run_sample(x, 6, 1.0, 3, 4)
    b = run_sample(x, 6, 1.0, 3, 4)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    c = run_sample(x, 6, 1.0, 3, 5)
    assert (c[0] != a[0]).any()
    dev = device()
    tok, _, _ = tav.tree_expand_topk(torch.from_numpy(x).to(dev), 6, 1.0)
    np.testing.assert_array_equal(to_numpy(tok), oracle.expand_topk(x, 6, 1.0)[0])
