"""Copy a seeded ``Workload`` to GPU tensors (plumbing only, no arithmetic)."""

from __future__ import annotations

import numpy as np
import torch


def _t(a: np.ndarray, device):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint64:
        a = a.view(np.int64)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(w, device="cuda", logits: bool = True) -> dict:
    """Dict of device tensors named like the C ABI's arguments."""
    d = {
        "parent": _t(w.parent, device),
        "token": _t(w.token, device),
        "q": _t(w.q, device),
        "k_tree": _t(w.k_tree, device),
        "v_tree": _t(w.v_tree, device),
        "k_cache": _t(w.k_cache, device),
        "v_cache": _t(w.v_cache, device),
        "block_table": _t(w.block_table, device),
        "prefix_len": _t(w.prefix_len, device),
    }
    if logits and w.target_logits is not None:
        d["target_logits"] = _t(w.target_logits, device)
        d["draft_logits"] = _t(w.draft_logits, device)
    return d


def to_numpy(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a
