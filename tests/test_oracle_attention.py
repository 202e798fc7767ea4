"""Pins for the oracle's tree attention (CPU only).

The oracle gathers the paged prefix, masks tree keys with the packed mask and
runs an explicit softmax. The pins reach the same numbers through
torch.nn.functional.scaled_dot_product_attention in float64 on dense,
unpaged tensors: causal attention for a chain, an explicit boolean mask from
DFS intervals for a general tree, and causal attention over the root-to-node
path alone. GQA uses SDPA's own ``enable_gqa`` head mapping.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_to_f32, make_workload


def _dense(w, b):
    """float64 torch tensors: q [Hq, N, D]; keys/values [Hkv, L+N, D]."""
    q = torch.from_numpy(bf16_to_f32(w.q[b]).astype(np.float64)).permute(1, 0, 2)
    kp = bf16_to_f32(w.k_prefix[b]).astype(np.float64)
    vp = bf16_to_f32(w.v_prefix[b]).astype(np.float64)
    kt = bf16_to_f32(w.k_tree[b]).astype(np.float64)
    vt = bf16_to_f32(w.v_tree[b]).astype(np.float64)
    k = torch.from_numpy(np.concatenate([kp, kt], 0)).permute(1, 0, 2)
    v = torch.from_numpy(np.concatenate([vp, vt], 0)).permute(1, 0, 2)
    return q, k, v


def _oracle(w):
    mask, _ = oracle.tree_mask(w.parent)
    return oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache,
                                 w.block_table, w.prefix_len, mask, scale=w.scale)


def _dfs_allowed(parent):
    n = len(parent)
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[parent[i]].append(i)
    tin, tout, clock = [0] * n, [0] * n, 0
    stack = [(0, False)]
    while stack:
        v, done = stack.pop()
        if done:
            tout[v] = clock
            continue
        tin[v] = clock
        clock += 1
        stack.append((v, True))
        stack.extend((c, False) for c in reversed(kids[v]))
    return np.array([[tin[j] <= tin[i] < tout[j] for j in range(n)] for i in range(n)])


@pytest.mark.parametrize("L,N,Hq,Hkv", [(37, 7, 4, 2), (0, 5, 2, 1), (64, 1, 8, 8), (200, 33, 6, 3)])
def test_chain_equals_causal_sdpa(L, N, Hq, Hkv):
    w = make_workload("tiny", N=N, Hq=Hq, Hkv=Hkv, D=64, L=(L, L), tree="chain",
                      with_logits=False, keep_dense=True, seed=11)
    out = _oracle(w)
    q, k, v = _dense(w, 0)
    # queries for the prefix positions are filler; only the last N rows are compared
    filler = torch.randn(Hq, L, w.D, dtype=torch.float64, generator=torch.Generator().manual_seed(0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.cat([filler, q], 1)[None], k[None], v[None], is_causal=True, enable_gqa=True)[0]
    ref = ref[:, L:, :].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,N,L", [(1, 40, 50), (2, 64, 16), (3, 100, 90)])
def test_random_tree_equals_sdpa_with_dfs_mask(seed, N, L):
    w = make_workload("tiny", N=N, Hq=4, Hkv=2, D=64, L=(L, L + 20), tree="random", B=2,
                      with_logits=False, keep_dense=True, seed=seed)
    out = _oracle(w)
    for b in range(w.B):
        Lb = int(w.prefix_len[b])
        q, k, v = _dense(w, b)
        allowed = np.ones((N, Lb + N), bool)
        allowed[:, Lb:] = _dfs_allowed(list(w.parent[b]))
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=torch.from_numpy(allowed), enable_gqa=True)[0]
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_node_equals_causal_attention_over_its_path():
    w = make_workload("tiny", N=30, Hq=2, Hkv=1, D=64, L=(45, 45), tree="random",
                      with_logits=False, keep_dense=True, seed=7)
    out = _oracle(w)
    q, k, v = _dense(w, 0)
    L = 45
    for i in [0, 5, 17, 29]:
        path = []
        j = i
        while j != -1:
            path.append(j)
            j = int(w.parent[0, j])
        path = path[::-1]
        keys = torch.cat([k[:, :L], k[:, [L + j for j in path]]], 1)
        vals = torch.cat([v[:, :L], v[:, [L + j for j in path]]], 1)
        # the node is the last query of a causal sequence prefix + path
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, i:i + 1][None], keys[None], vals[None])[0, :, 0]
        np.testing.assert_allclose(out[0, i], ref.numpy(), rtol=0, atol=1e-12)


def test_non_ancestor_kv_does_not_matter():
    w = make_workload("tiny", N=20, Hq=2, Hkv=1, D=64, L=(33, 33), tree="random",
                      with_logits=False, seed=5)
    base = _oracle(w)
    anc = oracle.ancestor_matrix(w.parent[0])
    i = 19
    others = [j for j in range(20) if not anc[i, j]]
    assert others
    w.k_tree[0, others] ^= np.uint16(0x1234)
    w.v_tree[0, others] ^= np.uint16(0x1234)
    np.testing.assert_array_equal(_oracle(w)[0, i], base[0, i])
    # an ancestor's V does matter
    w.v_tree[0, int(w.parent[0, i])] ^= np.uint16(0x0100)
    assert not np.array_equal(_oracle(w)[0, i], base[0, i])


def test_paged_gather_ignores_poisoned_slots():
    w = make_workload("tiny", N=5, L=(21, 21), with_logits=False, seed=3)
    out = _oracle(w)
    assert np.isfinite(out).all()
    # unused slots really are NaN-poisoned
    assert np.isnan(bf16_to_f32(w.k_cache)).any()


def test_bad_block_table_rejected():
    w = make_workload("tiny", N=5, L=(40, 40), with_logits=False, seed=3)
    w.block_table[0, 1] = w.k_cache.shape[0]
    with pytest.raises(ValueError):
        _oracle(w)
