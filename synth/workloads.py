"""Seeded workload generators.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed order,
so a (config, seed, overrides) triple always yields the same bits. Shapes and
value distributions follow the workloads the pages discuss: Llama-3-8B and
70B-shaped attention layers with grouped KV heads, paged KV in 16-token blocks,
64- to 128-node draft trees of depth 5 to 8 and width up to 4 (Sequoia's
depth/width table and the top-k branching rule on the jisaku.com glossary
page), and a 128256- or 151936-entry vocabulary.

Conventions shared with the library's C ABI:
  * ``parent[b][0] == -1`` and ``0 <= parent[b][i] < i`` (topological order);
  * ``token[b][i]`` is the draft token carried by node i (node 0 is the last
    committed token and is never tested);
  * K cache blocks are ``[num_blocks][Hkv][block][D]`` (token-major), V cache
    blocks are ``[num_blocks][Hkv][D][block]`` (feature-major);
  * ``block_table[b][j]`` is the physical block of logical block j, or -1.
"""

from __future__ import annotations

import dataclasses
import heapq
import os
from typing import Optional, Sequence

import numpy as np

BLOCK = 16
BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bf16 bit patterns (inputs are bf16; these helpers only produce/inspect bits)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# trees
# ----------------------------------------------------------------------------

def example_parent() -> np.ndarray:
    """The 5-node tree T0, A1, A2, B1, B2 of the radar-34b blog's mask example."""
    return np.array([-1, 0, 1, 0, 3], dtype=np.int32)


def chain_parent(n: int) -> np.ndarray:
    """A linear chain: node i's parent is i-1 (the gamma+1 = n case)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def random_parent(rng: np.random.Generator, n: int) -> np.ndarray:
    """Uniform random recursive tree: parent[i] uniform in [0, i)."""
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(0, i)
    return p


def _ranked_tokens(row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest raw logits, largest first, ties to lower id."""
    k = min(k, row.shape[0])
    cand = np.argpartition(-row, k - 1)[:k]
    order = np.lexsort((cand, -row[cand]))
    return cand[order].astype(np.int32)


def tokens_topk_for_parent(parent: np.ndarray, draft_rows: np.ndarray,
                           root_token: int) -> np.ndarray:
    """Give each node's children (ascending index) the top-ranked tokens of
    the parent's draft-logit row, in rank order (top-k branching)."""
    n = parent.shape[0]
    token = np.zeros(n, dtype=np.int32)
    token[0] = root_token
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[int(parent[i])].append(i)
    for u in range(n):
        if kids[u]:
            ranked = _ranked_tokens(draft_rows[u], len(kids[u]))
            for c, x in zip(kids[u], ranked):
                token[c] = x
    return token


def best_first_tree(draft_rows: np.ndarray, widths: Sequence[int], budget: int,
                    root_token: int):
    """Grow a draft tree best-first up to ``budget`` nodes.

    Node u proposes the ``widths[depth(u)]`` top tokens of its draft row. A
    candidate's score is its parent's score plus the gap between the token's
    draft logit and the largest logit of that row (a normaliser-free stand-in
    for cumulative draft log-probability). The best candidate becomes the next
    node (ties: earliest proposed), so ``parent[i] < i`` and node i owns row i.
    Returns (parent, token); fewer than ``budget`` nodes if the shape saturates.
    """
    parent = [-1]
    token = [int(root_token)]
    depth = [0]
    score = [0.0]
    heap = []
    seq = 0

    def propose(u):
        nonlocal seq
        d = depth[u]
        if d >= len(widths):
            return
        row = draft_rows[u]
        mx = float(row.max())
        for x in _ranked_tokens(row, widths[d]):
            heapq.heappush(heap, (-(score[u] + float(row[x]) - mx), seq, u, int(x), d + 1))
            seq += 1

    propose(0)
    while len(parent) < budget and heap:
        s, _, u, x, d = heapq.heappop(heap)
        parent.append(u)
        token.append(x)
        depth.append(d)
        score.append(-s)
        propose(len(parent) - 1)
    return np.array(parent, dtype=np.int32), np.array(token, dtype=np.int32)


# ----------------------------------------------------------------------------
# paged KV cache
# ----------------------------------------------------------------------------

def build_paged_cache(rng: np.random.Generator, k_prefix, v_prefix, n_nodes: int,
                      block: int = BLOCK, spare_blocks: int = 2, poison: bool = True):
    """Scatter dense per-sequence prefixes into a shuffled paged cache.

    Each sequence gets ``ceil((L_b + n_nodes) / block)`` logical blocks, enough
    to commit a whole tree path. Physical blocks are a seeded permutation.
    Slots that hold no prefix token are filled with bf16 NaN when ``poison`` is
    set, so any read of an unused slot shows up in the result.
    Returns (k_cache, v_cache, block_table).
    """
    B = len(k_prefix)
    Hkv, D = k_prefix[0].shape[1], k_prefix[0].shape[2]
    caps = [-(-(kp.shape[0] + n_nodes) // block) for kp in k_prefix]
    nblk = int(sum(caps)) + spare_blocks
    max_blocks = max(caps)
    perm = rng.permutation(nblk).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :caps[b]] = perm[off:off + caps[b]]
        off += caps[b]
    fill = BF16_NAN if poison else np.uint16(0)
    k_cache = np.full((nblk, Hkv, block, D), fill, dtype=np.uint16)
    v_cache = np.full((nblk, Hkv, D, block), fill, dtype=np.uint16)
    for b in range(B):
        L = k_prefix[b].shape[0]
        if L == 0:
            continue
        pos = np.arange(L)
        blk = table[b, pos // block]
        slot = pos % block
        k_cache[blk, :, slot, :] = k_prefix[b]
        v_cache[blk, :, :, slot] = v_prefix[b]
    return k_cache, v_cache, table


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    V: int
    block: int
    temperature: float
    philox_seed: int
    philox_offset: int
    parent: np.ndarray          # int32 [B, N]
    token: np.ndarray           # int32 [B, N]
    q: np.ndarray               # uint16 bf16 [B, N, Hq, D]
    k_tree: np.ndarray          # uint16 bf16 [B, N, Hkv, D]
    v_tree: np.ndarray          # uint16 bf16 [B, N, Hkv, D]
    prefix_len: np.ndarray      # int32 [B]
    k_cache: np.ndarray         # uint16 bf16 [nblk, Hkv, block, D]
    v_cache: np.ndarray         # uint16 bf16 [nblk, Hkv, D, block]
    block_table: np.ndarray     # int32 [B, max_blocks]
    target_logits: Optional[np.ndarray]  # float32 [B, N, V]
    draft_logits: Optional[np.ndarray]   # float32 [B, N, V]
    k_prefix: Optional[list] = None      # dense bf16 prefixes, [L_b, Hkv, D] each
    v_prefix: Optional[list] = None
    draft_noise: Optional[np.ndarray] = None   # the N(0, 1) draws behind draft - target
    widths: Optional[Sequence[int]] = None     # best-first widths per depth, if best-first

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_len.max()) if self.B else 0

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))


SWEEP_SIGMA = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "tests", "golden", "sweep_sigma.txt")


def sweep_sigma(accept: float) -> float:
    """Draft-noise sigma of the sweep workloads for a mean acceptance, read
    from the table that tests/golden/sweep_sigma.py computed with the
    oracle's softmax (this module computes no softmax)."""
    with open(SWEEP_SIGMA) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            a, s, _ = line.split()
            if abs(float(a) - accept) < 1e-9:
                return float(s)
    raise ValueError(f"no sweep sigma for acceptance {accept}")


# Named presets. Seeds are the preset's position in this table.
CONFIGS = {
    # 5-node worked-example tree, one head, head_dim 64, 128-token prefix.
    "tiny": dict(seed=0, B=1, N=5, Hq=1, Hkv=1, D=64, V=1000, L=(128, 128),
                 sigma_t=2.0, sigma_d=0.5, tree="example"),
    # Llama-3-8B-shaped layer, 64-node top-k tree of depth 5, widths 4,4,3,2,2.
    "llama8b": dict(seed=1, B=1, N=64, Hq=32, Hkv=8, D=128, V=128256, L=(4096, 4096),
                    sigma_t=3.0, sigma_d=1.0, tree="best_first", widths=(4, 4, 3, 2, 2)),
    # Llama-3-70B-shaped layer, batch 8, prefixes 6144..8192, depth 6 width <= 4.
    "llama70b": dict(seed=2, B=8, N=64, Hq=64, Hkv=8, D=128, V=128256, L=(6144, 8192),
                     sigma_t=3.0, sigma_d=1.0, tree="best_first", widths=(4,) * 6),
    # Batch-sweep shapes: 16-node tree (depth 4, width <= 3) and a gamma=5 chain;
    # the draft noise is set by the mean acceptance (0.5, 0.8 or 0.9).
    "sweep_tree16": dict(seed=3, B=1, N=16, Hq=32, Hkv=8, D=128, V=128256, L=(2048, 2048),
                         sigma_t=3.0, accept=0.8, tree="best_first", widths=(3, 3, 3, 3)),
    "sweep_chain6": dict(seed=3, B=1, N=6, Hq=32, Hkv=8, D=128, V=128256, L=(2048, 2048),
                         sigma_t=3.0, accept=0.8, tree="chain"),
    # One GPU's share of the 70B-shaped layer under 8-way tensor parallelism
    # over KV heads: one KV head and its 8 query heads, the rest as the 70B
    # layer (seeded as it, not by position).
    "llama70b_tp8": dict(seed=2, B=8, N=64, Hq=8, Hkv=1, D=128, V=128256, L=(6144, 8192),
                         sigma_t=3.0, sigma_d=1.0, tree="best_first", widths=(4,) * 6),
    # Long context: 70B-shaped layer, 32K paged prefix, 128-node depth-8 tree.
    "long": dict(seed=4, B=4, N=128, Hq=64, Hkv=8, D=128, V=151936, L=(32768, 32768),
                 sigma_t=3.0, sigma_d=0.7, tree="best_first", widths=(4,) * 8),
}


def make_workload(name: str, *, seed: Optional[int] = None, with_logits: bool = True,
                  keep_dense: bool = False, poison: bool = True, keep_noise: bool = False,
                  **over) -> Workload:
    """Build a preset, optionally overriding any of its fields.

    Overrides: B, N, Hq, Hkv, D, V, L=(lo, hi) inclusive prefix-length range,
    sigma_t, sigma_d, tree ('example' | 'chain' | 'random' | 'best_first'),
    widths, temperature, philox_seed, philox_offset, accept (the sweep
    presets' mean acceptance, which sets sigma_d).
    """
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if cfg.get("accept") is not None and "sigma_d" not in over:
        cfg["sigma_d"] = sweep_sigma(float(cfg["accept"]))
    seed = cfg["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D, V = (int(cfg[k]) for k in ("B", "N", "Hq", "Hkv", "D", "V"))
    lo, hi = cfg["L"]
    T = float(cfg.get("temperature", 1.0))
    tree = cfg["tree"]

    # Logits: target ~ N(0, sigma_t^2); draft = target + N(0, sigma_d^2).
    tl = dl = None
    if with_logits or tree == "best_first":
        tl = rng.standard_normal((B, N, V), dtype=np.float32)
        tl *= np.float32(cfg["sigma_t"])
        dl = rng.standard_normal((B, N, V), dtype=np.float32)
        noise = dl.copy() if keep_noise else None
        dl *= np.float32(cfg["sigma_d"])
        dl += tl

    parent = np.empty((B, N), dtype=np.int32)
    token = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        root_tok = int(rng.integers(0, V))
        if tree == "example":
            assert N == 5
            p = example_parent()
        elif tree == "chain":
            p = chain_parent(N)
        elif tree == "random":
            p = random_parent(rng, N)
        elif tree == "best_first":
            p, t = best_first_tree(dl[b], cfg["widths"], N, root_tok)
            if p.shape[0] != N:
                raise ValueError(f"tree saturated at {p.shape[0]} < {N} nodes")
            parent[b] = p
            token[b] = t
            continue
        else:
            raise ValueError(tree)
        parent[b] = p
        if dl is not None:
            token[b] = tokens_topk_for_parent(p, dl[b], root_tok)
        else:
            token[b] = rng.integers(0, V, size=N)
            token[b, 0] = root_tok

    q = bf16_bits(rng.standard_normal((B, N, Hq, D), dtype=np.float32))
    k_tree = bf16_bits(rng.standard_normal((B, N, Hkv, D), dtype=np.float32))
    v_tree = bf16_bits(rng.standard_normal((B, N, Hkv, D), dtype=np.float32))
    prefix_len = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    k_prefix = [bf16_bits(rng.standard_normal((int(L), Hkv, D), dtype=np.float32))
                for L in prefix_len]
    v_prefix = [bf16_bits(rng.standard_normal((int(L), Hkv, D), dtype=np.float32))
                for L in prefix_len]
    k_cache, v_cache, table = build_paged_cache(rng, k_prefix, v_prefix, N, poison=poison)

    return Workload(
        name=name, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, block=BLOCK, temperature=T,
        philox_seed=int(cfg.get("philox_seed", 0)), philox_offset=int(cfg.get("philox_offset", 0)),
        parent=parent, token=token, q=q, k_tree=k_tree, v_tree=v_tree,
        prefix_len=prefix_len, k_cache=k_cache, v_cache=v_cache, block_table=table,
        target_logits=tl if with_logits else None, draft_logits=dl if with_logits else None,
        k_prefix=k_prefix if keep_dense else None, v_prefix=v_prefix if keep_dense else None,
        draft_noise=noise if (keep_noise and with_logits) else None,
        widths=tuple(cfg["widths"]) if tree == "best_first" else None,
    )


def with_acceptance(w: Workload, accept: float) -> Workload:
    """The same workload with the draft noise rescaled to the sweep sigma of
    ``accept`` (draft = target + sigma * the same N(0, 1) draws), and the tree
    and tokens rebuilt from the new draft rows as ``make_workload`` builds
    them: equal, bit for bit, to ``make_workload`` of that acceptance. Needs
    a workload made with ``keep_noise=True``."""
    if w.draft_noise is None:
        raise ValueError("workload was made without keep_noise")
    dl = w.draft_noise.copy()
    dl *= np.float32(sweep_sigma(accept))
    dl += w.target_logits
    parent = np.empty_like(w.parent)
    token = np.empty_like(w.token)
    for b in range(w.B):
        root_tok = int(w.token[b, 0])
        if w.widths is not None:
            p, t = best_first_tree(dl[b], w.widths, w.N, root_tok)
            if p.shape[0] != w.N:
                raise ValueError(f"tree saturated at {p.shape[0]} < {w.N} nodes")
            parent[b], token[b] = p, t
        else:
            parent[b] = w.parent[b]
            token[b] = tokens_topk_for_parent(w.parent[b], dl[b], root_tok)
    return dataclasses.replace(w, parent=parent, token=token, draft_logits=dl)


def slice_batch(w: Workload, B: int) -> Workload:
    """The first B sequences of a workload (the paged caches are shared)."""
    cut = lambda a: None if a is None else a[:B]
    return dataclasses.replace(
        w, B=B, parent=w.parent[:B], token=w.token[:B], q=w.q[:B], k_tree=w.k_tree[:B],
        v_tree=w.v_tree[:B], prefix_len=w.prefix_len[:B], block_table=w.block_table[:B],
        target_logits=cut(w.target_logits), draft_logits=cut(w.draft_logits),
        draft_noise=cut(w.draft_noise),
        k_prefix=None if w.k_prefix is None else w.k_prefix[:B],
        v_prefix=None if w.v_prefix is None else w.v_prefix[:B])


def gather_nodes(w: Workload, parent, token, src) -> Workload:
    """A workload whose trees are given (parent, token int [B, M]) and whose
    node j of sequence b takes the rows of node src[b, j] of `w` (Q, the
    tree's K/V, both logits). For trees built elsewhere over w's rows; the
    prefix, caches and block table are w's."""
    src = np.asarray(src, dtype=np.int64)
    B, M = src.shape
    take = lambda a: None if a is None else np.ascontiguousarray(
        np.take_along_axis(a, src.reshape((B, M) + (1,) * (a.ndim - 2)), axis=1))
    return dataclasses.replace(
        w, N=M, parent=np.ascontiguousarray(parent, dtype=np.int32),
        token=np.ascontiguousarray(token, dtype=np.int32), q=take(w.q), k_tree=take(w.k_tree),
        v_tree=take(w.v_tree), target_logits=take(w.target_logits),
        draft_logits=take(w.draft_logits), draft_noise=take(w.draft_noise), widths=None)


def slice_nodes(w: Workload, n: int) -> Workload:
    """The first n nodes of every tree (a subtree: nodes are numbered
    topologically), with their rows; n = 1 leaves the root alone, a decode
    step's shape."""
    cut = lambda a: None if a is None else np.ascontiguousarray(a[:, :n])
    return dataclasses.replace(
        w, N=n, parent=cut(w.parent), token=cut(w.token), q=cut(w.q), k_tree=cut(w.k_tree),
        v_tree=cut(w.v_tree), target_logits=cut(w.target_logits),
        draft_logits=cut(w.draft_logits), draft_noise=cut(w.draft_noise))
