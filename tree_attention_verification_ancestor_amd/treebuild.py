"""Tree construction from draft rows with the library's calls.

jisaku.com glossary, tree-topology strategies: entropy-based branching gives
uncertain nodes more branches, and the budget-constrained strategy caps the
node count. entropy_tree grows candidate trees level by level over a batch
of draft rows and keeps the budget's best nodes:

* level 0: the root (row 0) takes `root_width` children;
* every later level: tree_expand_topk over the frontier's draft rows, then
  tree_widths_by_entropy (the frontier ranked by entropy, widths in
  [w_min, w_max]); each node's children are its top tokens up to its width;
* candidate node i of a sequence takes draft row i (children are numbered
  in frontier order, then by rank, so the numbering stays topological);
* tree_select_topm keeps the `budget` nodes of largest cumulative log q.

All arithmetic runs in the library's kernels; between levels only the
widths and the top tokens (a few KB) cross to the host to number the
children. The rank widths of a level sum to the same count in every
sequence, so the batch stays rectangular.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (new_flags, tree_expand_topk, tree_select_topm, tree_widths_by_entropy)


def entropy_tree(draft, temperature: float, depth: int, root_width: int, w_min: int, w_max: int,
                 budget: int, dev_flags=None):
    """draft: fp32 [B, R, V] device tensor of candidate rows. Returns
    (parent, token, src) int32 device tensors [B, M] (M = min(budget,
    candidates); src = each kept node's row) and the candidates per level."""
    if draft.dim() != 3:
        raise ValueError("draft must be [B, R, V]")
    B, R, V = draft.shape
    dev = draft.device
    flags = new_flags(dev) if dev_flags is None else dev_flags
    k = max(root_width, w_max)
    parent = [[-1] for _ in range(B)]
    token = [[0] for _ in range(B)]
    logq = [[0.0] for _ in range(B)]
    start, F, sizes = 0, 1, [1]
    for level in range(depth):
        rows = draft[:, start:start + F, :].reshape(B * F, V).contiguous()
        tok, lq, ent = tree_expand_topk(rows, k, temperature, dev_flags=flags)
        if level == 0:
            widths = np.full((B, F), root_width, np.int64)
        else:
            widths = tree_widths_by_entropy(ent.view(B, F), w_min, w_max,
                                            dev_flags=flags).cpu().numpy()
        tok = tok.cpu().numpy().reshape(B, F, k)
        lq = lq.cpu().numpy().reshape(B, F, k)
        total = min(int(widths[0].sum()), R - (start + F))
        if total <= 0:
            break
        for b in range(B):
            n = 0
            for i in range(F):
                for r in range(int(widths[b, i])):
                    if n < total:
                        parent[b].append(start + i)
                        token[b].append(int(tok[b, i, r]))
                        logq[b].append(float(lq[b, i, r]))
                        n += 1
        start, F = start + F, total
        sizes.append(total)
    nc = start + F
    t = lambda a, dt: torch.tensor(np.array(a), dtype=dt, device=dev)
    op, ot, src = tree_select_topm(t(parent, torch.int32), t(token, torch.int32),
                                   t(logq, torch.float64), min(budget, nc), dev_flags=flags)
    return op, ot, src, sizes
