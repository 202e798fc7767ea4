"""Tree attention over a paged prefix, the plain definition in float64.

What it computes:
  * LLM Primer VI ch. 9, section 9.1: the target runs one forward pass over the
    committed prefix with the candidates appended, so every candidate position
    is scored in the same pass.
  * jisaku.com glossary "Tree-based speculative decoding", tree-attention
    section: a node attends only along its own root-to-node path; this extends
    the usual causal mask. The radar-34b blog's section 3 matrix is the
    5-node example.
  * radar-34b blog section 5 and the glossary's KV-cache section: the prefix
    lives in a paged KV cache addressed through a block table.

Readings where the pages are silent: every node sees the whole committed
prefix [0, L_b); scores are scaled by ``scale`` (1/sqrt(D) by default); query
head h reads KV head h // (Hq / Hkv); inputs are bf16 and are widened exactly.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def gather_prefix(k_cache, v_cache, block_table_row, L: int, block: int):
    """Dense [L, Hkv, D] prefix K and V read through one block-table row."""
    if L == 0:
        Hkv, D = k_cache.shape[1], k_cache.shape[3]
        return np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D))
    pos = np.arange(L)
    logical = pos // block
    if logical.max() >= block_table_row.shape[0]:
        raise ValueError("prefix longer than the block table")
    blk = block_table_row[logical]
    if (blk < 0).any() or (blk >= k_cache.shape[0]).any():
        raise ValueError("block table entry outside the cache")
    slot = pos % block
    K = bf16_bits_to_f64(k_cache[blk, :, slot, :])      # K blocks: [blk][h][slot][d]
    V = bf16_bits_to_f64(v_cache[blk, :, :, slot])      # V blocks: [blk][h][d][slot]
    return K, V


def unpack_mask(mask_row: np.ndarray, N: int) -> np.ndarray:
    """Boolean [N, N] from packed uint64 words [N, W] (bit j%64 of word j//64)."""
    j = np.arange(N)
    words = mask_row[:, j // 64]
    return ((words >> (j % 64).astype(np.uint64)) & np.uint64(1)).astype(bool)


def tree_attention(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len, mask,
                   scale=None, block: int = 16, batches=None, kv_heads=None):
    """float64 [B, N, Hq, D] attention output.

    q [B,N,Hq,D], k_tree/v_tree [B,N,Hkv,D], caches as described in the module
    header (all bf16 bits); block_table [B, max_blocks]; prefix_len [B];
    mask uint64 [B,N,W]. ``batches``/``kv_heads`` restrict the work to a subset
    (other entries are left NaN), for sampled checks at full size.
    """
    B, N, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, N, Hq, D), np.nan)
    for b in (range(B) if batches is None else batches):
        L = int(prefix_len[b])
        Kp, Vp = gather_prefix(k_cache, v_cache, block_table[b], L, block)
        allowed = unpack_mask(mask[b], N)                    # [N (query), N (key)]
        for kv in (range(Hkv) if kv_heads is None else kv_heads):
            K = np.concatenate([Kp[:, kv, :], bf16_bits_to_f64(k_tree[b, :, kv, :])], axis=0)
            V = np.concatenate([Vp[:, kv, :], bf16_bits_to_f64(v_tree[b, :, kv, :])], axis=0)
            for h in range(kv * G, (kv + 1) * G):
                Q = bf16_bits_to_f64(q[b, :, h, :])           # [N, D]
                s = (Q @ K.T) * scale                          # [N, L + N]
                s[:, L:][~allowed] = -np.inf                   # tree keys: ancestors and self only
                s -= s.max(axis=1, keepdims=True)
                e = np.exp(s)
                p = e / e.sum(axis=1, keepdims=True)
                out[b, :, h, :] = p @ V
    return out
