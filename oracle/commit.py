"""KV commit of the accepted path, the plain definition.

radar-34b blog section 5 (KV-cache management) and the jisaku.com glossary's
KV-cache section: after verification only the accepted path's entries are
kept; rejected branches are pruned and the cache is rolled back to the
accepted length, with paged blocks making this cheap.

Reading: accepted node path[t] (t = 0..m, the root first) becomes the token at
position L_b + t of sequence b, stored in slot pos % block of physical block
block_table[b][pos // block]; the new length is L_b + m + 1. Nothing else in
the cache changes.
"""

from __future__ import annotations

import numpy as np


def kv_commit(k_tree, v_tree, path, n_accepted, block_table, prefix_len, k_cache, v_cache,
              block: int = 16):
    """Returns (k_cache', v_cache', commit_slots int32 [B, N], new_prefix_len int32 [B]).

    The input caches are not modified; copies are returned. commit_slots[b][t]
    is the flat slot index blk * block + pos % block, or -1 beyond the path.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    B, N = path.shape
    slots = np.full((B, N), -1, dtype=np.int32)
    new_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(prefix_len[b])
        m = int(n_accepted[b])
        for t in range(m + 1):
            node = int(path[b, t])
            pos = L + t
            logical = pos // block
            if logical >= block_table.shape[1]:
                raise ValueError("block table too short for the accepted path")
            blk = int(block_table[b, logical])
            if not (0 <= blk < k_cache.shape[0]):
                raise ValueError("block table entry outside the cache")
            s = pos % block
            k_out[blk, :, s, :] = k_tree[b, node]          # K blocks: [blk][h][slot][d]
            v_out[blk, :, :, s] = v_tree[b, node]          # V blocks: [blk][h][d][slot]
            slots[b, t] = blk * block + s
        new_len[b] = L + m + 1
    return k_out, v_out, slots, new_len


def _slot(block_table, b, pos, nblk, block):
    logical = pos // block
    if logical >= block_table.shape[1]:
        raise ValueError("block table too short for the tree")
    blk = int(block_table[b, logical])
    if not (0 <= blk < nblk):
        raise ValueError("block table entry outside the cache")
    return blk, pos % block


def kv_commit_inplace(path, n_accepted, block_table, prefix_len, k_cache, v_cache,
                      block: int = 16):
    """Zero-copy rollback: the tree's rows already sit in the cache.

    radar-34b blog section 5: engines branch and roll back the tree through
    block-table operations without copying; jisaku.com glossary, KV-cache
    section: entries off the accepted path are pruned and the cache is rolled
    back to the right position. Reading: node i of sequence b was written at
    position L_b + i. Afterwards position L_b + t holds what position
    L_b + path[t] held (t = 0..m), every row read before any is written; the
    length becomes L_b + m + 1, and the positions past it are abandoned, not
    freed or cleared. Nothing else changes.

    Returns (k_cache', v_cache', commit_slots int32 [B, N], new_prefix_len).
    """
    k_old = np.asarray(k_cache)
    v_old = np.asarray(v_cache)
    k_out = np.array(k_old, copy=True)
    v_out = np.array(v_old, copy=True)
    B, N = path.shape
    nblk = k_old.shape[0]
    slots = np.full((B, N), -1, dtype=np.int32)
    new_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(prefix_len[b])
        m = int(n_accepted[b])
        _slot(block_table, b, L + N - 1, nblk, block)        # the tree fits the table
        for t in range(m + 1):
            db, ds = _slot(block_table, b, L + t, nblk, block)
            sb, ss = _slot(block_table, b, L + int(path[b, t]), nblk, block)
            k_out[db, :, ds, :] = k_old[sb, :, ss, :]
            v_out[db, :, :, ds] = v_old[sb, :, :, ss]
            slots[b, t] = db * block + ds
        new_len[b] = L + m + 1
    return k_out, v_out, slots, new_len
