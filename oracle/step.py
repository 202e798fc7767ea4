"""The whole verification step, composed from the oracle's parts.

Order follows the pipeline table at the top of the radar-34b blog (tree mask,
one verification forward over all candidates, rejection sampling, rollback):
mask -> tree attention -> walk -> KV commit.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .attention import tree_attention
from .commit import kv_commit
from .mask import tree_mask
from .sampling import WalkResult, verify_walk


@dataclasses.dataclass
class StepResult:
    mask: np.ndarray
    depth: np.ndarray
    attn_out: np.ndarray
    walk: WalkResult
    k_cache: np.ndarray
    v_cache: np.ndarray
    commit_slots: np.ndarray
    new_prefix_len: np.ndarray


def verify_step_ref(w, batches=None, kv_heads=None) -> StepResult:
    """Run the oracle over a ``synth.Workload``.

    ``batches``/``kv_heads`` restrict the attention part to a sample (the walk
    and commit always run on every sequence)."""
    mask, depth = tree_mask(w.parent)
    out = tree_attention(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache, w.block_table,
                         w.prefix_len, mask, scale=w.scale, block=w.block,
                         batches=batches, kv_heads=kv_heads)
    walk = verify_walk(w.target_logits, w.draft_logits, w.parent, w.token, w.temperature,
                       w.philox_seed, w.philox_offset)
    k2, v2, slots, new_len = kv_commit(w.k_tree, w.v_tree, walk.path, walk.n_accepted,
                                       w.block_table, w.prefix_len, w.k_cache, w.v_cache,
                                       block=w.block)
    return StepResult(mask, depth, out, walk, k2, v2, slots, new_len)
