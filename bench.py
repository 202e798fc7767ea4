"""Benchmark of the tree-verification step on one MI355X.

A step is one pass of the whole path over one batch, chained on one stream
with no host synchronisation: tree_attn_verify_tree (one attention layer, the
ancestor mask built from parent[] in the same launch and written out) and
spec_verify_sample_commit (the rejection-sampling walk, each sequence's
accepted path committed to the paged cache by the walk's own workgroups).
The same step as four calls (tree_mask_build, tree_attn_verify,
spec_verify_sample, kv_commit_path) is timed beside it for the per-call
breakdown. Inputs are seeded synthetic data already resident in HBM.

The headline workload is the Llama-3-70B-shaped layer: batch 8, 64-node trees
(depth 6, width 4), 64 query / 8 KV heads, head_dim 128, paged prefixes of
6144..8192 tokens, a 128256-entry vocabulary. Three copies of its paged caches
rotate across steps so the 256 MB last-level cache cannot hold the step's KV
working set. Its line carries the attention launch's roofline (events on the
launch stream inside the timed region; HBM traffic from the rocprofv3
counter record under profiles/ while that record matches the kernel source),
the CPU oracle's rate on this host, per-stage percentiles, the acceptance over
many Philox offsets, and timed legs of the other calls.

`configs` reports the other workloads the same way, each step timed on its
own with a 512 MB write between steps (so the last-level cache starts cold,
as it would after a model's other layers): the tiny worked example, the
Llama-3-8B layer at batch 1, the batch sweep (batch 1..128, a 16-node tree
against a 6-node chain, mean acceptance 0.5 / 0.8 / 0.9) and the 32K-token
long context. Each has step us, nodes/s, emitted tokens per step, realised
acceptance, the attention roofline and the oracle's rate on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config llama70b] [--no-cpu]
                    [--offsets 1000] [--no-configs] [--config-steps 20]
    python bench.py --copy-calibration     # a plain copy of known size, for the counters
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "tree_attn_llama70b_hbm_traffic.txt")
COPY_BYTES = 1 << 30           # each of the calibration copy's read and write
FLUSH_BYTES = 512 << 20        # written between the configs' steps
SWEEP_BATCHES = (1, 4, 16, 64, 128)
SWEEP_ACCEPTS = (0.5, 0.8, 0.9)
# Llama-3-8B, the sweep's shape: 32 layers of 4096-wide projections (q, k,
# v, o: 4096 x (4096 + 1024 + 1024 + 4096); MLP 3 x 4096 x 14336) and a
# 128256 x 4096 vocabulary head
LAYERS_8B = 32
LAYER_PARAMS_8B = 4096 * (4096 + 1024 + 1024 + 4096) + 3 * 4096 * 14336
HEAD_PARAMS_8B = 128256 * 4096
STAGES_UNFUSED = ["tree_mask_build", "tree_attn_verify", "spec_verify_sample", "kv_commit_path"]
STAGES = ["tree_attn_verify_tree", "spec_verify_sample_commit"]


# ---------------------------------------------------------------------------
# algorithmic work

def workload_desc(w) -> str:
    return (f"{w.name}: B={w.B}, N={w.N}-node trees, {w.Hq}/{w.Hkv} heads, D={w.D}, "
            f"paged prefix {int(w.prefix_len.min())}..{int(w.prefix_len.max())} "
            f"(block {w.block}), vocab {w.V}, T={w.temperature}")


def attention_work(w, depth):
    """Algorithmic bytes and FLOPs of one tree_attn_verify launch."""
    L = int(w.prefix_len.sum())
    kv = L * w.Hkv * w.D * 2 * 2                       # prefix K and V, bf16, read once
    q = w.B * w.N * w.Hq * w.D * 2
    tree = w.B * w.N * w.Hkv * w.D * 2 * 2
    out = w.B * w.N * w.Hq * w.D * 4
    small = w.B * w.N * ((w.N + 63) // 64) * 8 + w.block_table.size * 4
    anc = int((depth + 1).sum())                        # sum over nodes of |ancestors or self|
    flops = 4 * w.Hq * w.D * (w.N * L + anc)
    return kv + q + tree + out + small, flops


def sampler_bytes(w, path, n_acc):
    """Target row of every visited node, plus the draft row of every visited
    node that has children (the rows the walk must read at least once)."""
    rows = 0
    for b in range(w.B):
        kids = set(int(x) for x in w.parent[b, 1:])
        for t in range(int(n_acc[b]) + 1):
            u = int(path[b, t])
            rows += 1 + (1 if u in kids else 0)
    return rows * w.V * 4 + w.B * w.N * 4 * 4


def commit_bytes(w, n_acc):
    return int((n_acc + 1).sum()) * w.Hkv * w.D * 2 * 2 * 2


def roofline(bytes_, flops, seconds):
    """The binding roofline of a launch of this work taking `seconds`."""
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4)}
    ach = bytes_ / seconds / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4)}


def acceptance_stats(w, paths, naccs):
    """Over Philox offsets: mean accepted per sequence, mean emitted tokens
    per step (accepted + 1 per sequence), the realised acceptance (children
    accepted / children tested: a child after its earlier siblings' rejection
    is one more test), and the mean rows the walk must read."""
    B, N = w.parent.shape
    rank = np.zeros((B, N), np.int64)       # position among its parent's children, from 1
    nkids = np.zeros((B, N), np.int64)
    for b in range(B):
        for i in range(1, N):
            u = int(w.parent[b, i])
            nkids[b, u] += 1
            rank[b, i] = nkids[b, u]
    tests = acc = 0
    for o in range(len(naccs)):
        for b in range(B):
            m = int(naccs[o, b])
            p = paths[o, b, :m + 1]
            tests += int(rank[b, p[1:]].sum()) + int(nkids[b, p[-1]])
            acc += m
    samp = float(np.mean([sampler_bytes(w, paths[o], naccs[o]) for o in range(len(naccs))]))
    comm = float(np.mean([commit_bytes(w, naccs[o]) for o in range(len(naccs))]))
    return {"offsets": int(len(naccs)),
            "mean_accepted_per_seq": round(float(naccs.mean()), 4),
            "mean_emitted_per_step": round(float((naccs + 1).sum(axis=1).mean()), 3),
            "realised_acceptance": round(acc / tests, 4) if tests else None,
            "mean_sampler_bytes": round(samp), "mean_commit_bytes": round(comm)}


def rank_acceptance(w, paths, naccs, K=16):
    """Acceptance rate of the k-th child by rank (k = 1..K): of the times the
    walk tried a node's k-th child, the share it accepted."""
    B, N = w.parent.shape
    rank = np.zeros((B, N), np.int64)
    kids = [[[] for _ in range(N)] for _ in range(B)]
    for b in range(B):
        for i in range(1, N):
            u = int(w.parent[b, i])
            kids[b][u].append(i)
            rank[b, i] = len(kids[b][u])
    tried = np.zeros(K + 1)
    took = np.zeros(K + 1)
    for o in range(len(naccs)):
        for b in range(B):
            m = int(naccs[o, b])
            p = paths[o, b, :m + 1]
            for t in range(m + 1):
                u = int(p[t])
                ch = kids[b][u]
                if not ch:
                    continue
                r_acc = int(rank[b, p[t + 1]]) if t < m else 0
                n_try = r_acc if r_acc else len(ch)
                for r in range(1, min(n_try, K) + 1):
                    tried[r] += 1
                    took[r] += 1 if r == r_acc else 0
    return [float(took[r] / tried[r]) if tried[r] else 0.0 for r in range(1, K + 1)], tried[1:]


def pct(a):
    return {"p10": round(float(np.percentile(a, 10)) * 1e3, 2),
            "p50": round(float(np.percentile(a, 50)) * 1e3, 2),
            "p90": round(float(np.percentile(a, 90)) * 1e3, 2)}


# ---------------------------------------------------------------------------
# the step on the GPU

class StepRunner:
    """A step over one workload as two fused calls (the default) or as the
    four separate calls, pre-marshalled, with `copies` copies of the paged
    caches to rotate through."""

    def __init__(self, w, dev, copies=1):
        import torch

        import tree_attention_verification_ancestor_amd as tav
        from synth.device import upload

        self.w, self.dev, self.torch, self.tav = w, dev, torch, tav
        d = upload(w, dev)
        self.d = d
        self.copies = [(d["k_cache"], d["v_cache"])]
        for _ in range(copies - 1):
            self.copies.append((d["k_cache"].clone(), d["v_cache"].clone()))
        B, N, V = w.B, w.N, w.V
        self.flags = tav.new_flags(dev)
        self.mask = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=dev)
        self.depth = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, N, w.Hq, w.D), dtype=torch.float32, device=dev)
        self.ws_a = tav.new_attn_workspace(B, N, w.Hq, w.Hkv, w.D, w.max_prefix_len, dev)
        self.ws_s = tav.new_sampler_workspace(B, N, V, dev)
        self.path = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
        self.toks = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.slots = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.new_len = torch.empty((B,), dtype=torch.int32, device=dev)
        self.stream = torch.cuda.current_stream()
        s = self.stream
        # one checked call of each entry point, then pre-marshalled calls
        tav.tree_mask_build(d["parent"], self.mask, self.depth, self.flags, s)
        tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], self.copies[0][0],
                             self.copies[0][1], d["block_table"], d["prefix_len"],
                             w.max_prefix_len, self.mask, w.scale, self.out, self.ws_a,
                             self.flags, s)
        tav.spec_verify_sample(d["target_logits"], d["draft_logits"], d["parent"], d["token"],
                               w.temperature, w.philox_seed, w.philox_offset, self.path,
                               self.n_acc, self.toks, self.ws_s, self.flags, s)
        tav.kv_commit_path(d["k_tree"], d["v_tree"], self.path, self.n_acc, d["block_table"],
                           d["prefix_len"], self.copies[0][0], self.copies[0][1], self.slots,
                           self.new_len, self.flags, s)
        torch.cuda.synchronize()
        nblk, maxb = int(w.k_cache.shape[0]), int(w.block_table.shape[1])
        self.calls_unfused = []
        self.calls = []
        for kc, vc in self.copies:
            self.calls.append((
                tav.prepare("tree_attn_verify_tree", d["q"], d["k_tree"], d["v_tree"], kc, vc,
                            nblk, d["block_table"], maxb, d["prefix_len"], w.max_prefix_len,
                            d["parent"], self.mask, self.depth, B, N, w.Hq, w.Hkv, w.D, w.block,
                            w.scale, self.out, self.ws_a, self.ws_a.numel(), self.flags, s),
                tav.prepare("spec_verify_sample_commit", d["target_logits"], d["draft_logits"],
                            d["parent"], d["token"], B, N, V, w.temperature, w.philox_seed,
                            w.philox_offset, 0, self.path, self.n_acc, self.toks, d["k_tree"],
                            d["v_tree"], nblk, d["block_table"], maxb, d["prefix_len"], kc, vc,
                            w.Hkv, w.D, w.block, self.slots, self.new_len, self.ws_s,
                            self.ws_s.numel(), self.flags, s),
            ))
            self.calls_unfused.append((
                tav.prepare("tree_mask_build", d["parent"], B, N, self.mask, self.depth,
                            self.flags, s),
                tav.prepare("tree_attn_verify", d["q"], d["k_tree"], d["v_tree"], kc, vc, nblk,
                            d["block_table"], maxb, d["prefix_len"], w.max_prefix_len,
                            self.mask, B, N, w.Hq, w.Hkv, w.D, w.block, w.scale, self.out,
                            self.ws_a, self.ws_a.numel(), self.flags, s),
                tav.prepare("spec_verify_sample", d["target_logits"], d["draft_logits"],
                            d["parent"], d["token"], B, N, V, w.temperature, w.philox_seed,
                            w.philox_offset, self.path, self.n_acc, self.toks, self.ws_s,
                            self.ws_s.numel(), self.flags, s),
                tav.prepare("kv_commit_path", d["k_tree"], d["v_tree"], self.path, self.n_acc,
                            nblk, d["block_table"], maxb, d["prefix_len"], kc, vc, B, N, w.Hkv,
                            w.D, w.block, self.slots, self.new_len, self.flags, s),
            ))
        self.i = 0

    def step(self, ev=None, attn_ev=None, unfused=False):
        """One step; ev: events before and after each call; attn_ev: events
        around the attention launch."""
        calls = self.calls_unfused if unfused else self.calls
        c = calls[self.i % len(calls)]
        self.i += 1
        attn = 1 if unfused else 0
        if ev:
            ev[0].record(self.stream)
        for k in range(len(c)):
            if attn_ev and k == attn:
                attn_ev[0].record(self.stream)
            c[k]()
            if attn_ev and k == attn:
                attn_ev[1].record(self.stream)
            if ev:
                ev[k + 1].record(self.stream)

    def ramp(self, seconds=0.3):
        """Steps until `seconds` have passed: the device reaches its working
        clock before anything is timed."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                self.step()
            self.torch.cuda.synchronize()

    def events(self, n):
        E = self.torch.cuda.Event
        return [[E(enable_timing=True) for _ in range(n)]]

    def check(self):
        self.torch.cuda.synchronize()
        f = int(self.flags.item())
        assert f == 0, f"device flags {f:#x}"

    def offsets(self, n):
        """The walk at Philox offsets 0..n-1 (outside every timed region)."""
        torch, tav, d, w = self.torch, self.tav, self.d, self.w
        paths = torch.empty((n, w.B, w.N), dtype=torch.int32, device=self.dev)
        naccs = torch.empty((n, w.B), dtype=torch.int32, device=self.dev)
        toks = torch.empty((n, w.B, w.N), dtype=torch.int32, device=self.dev)
        for o in range(n):
            tav.spec_verify_sample(d["target_logits"], d["draft_logits"], d["parent"], d["token"],
                                   w.temperature, w.philox_seed, o, paths[o], naccs[o], toks[o],
                                   self.ws_s, self.flags, self.stream)
        self.check()
        from synth.device import to_numpy
        return to_numpy(paths), to_numpy(naccs)

    def cold_steps(self, n, warmup, flush, unfused=False):
        """n steps, each after a write of `flush` (the last-level cache cold),
        with events between the calls: per-step and per-call ms."""
        torch = self.torch
        k = 4 if unfused else 2
        for _ in range(warmup):
            self.step(unfused=unfused)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(k + 1)] for _ in range(n)]
        for e in evs:
            flush.fill_(1)
            self.step(ev=e, unfused=unfused)
        self.check()
        stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(k)] for e in evs])
        step = np.array([e[0].elapsed_time(e[k]) for e in evs])
        return step, stage


def run_headline(args, w):
    """The headline workload: timed region, stage pass, acceptance and the
    other calls' legs."""
    import torch

    import tree_attention_verification_ancestor_amd as tav
    from synth.device import to_numpy

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    r = StepRunner(w, dev, copies=args.cache_copies)
    B, N, V = w.B, w.N, w.V
    d, stream, flags = r.d, r.stream, r.flags
    r.ramp()
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps between two synchronised events;
    # the attention launch of every step is bracketed by events on its stream
    attn_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        r.step(attn_ev=attn_evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    attn_ms = np.array([e[0].elapsed_time(e[1]) for e in attn_evs])

    # per-call times with events on the launch stream (a second pass), and
    # the same step as four separate calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        r.step(ev=evs[i])
    r.check()
    stage = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(2)] for e in evs])
    out = dict(ms_step=ms_step, ms_attn=float(attn_ms.mean()), attn_all=attn_ms,
               stage_ms=stage.mean(axis=0), stage_all=stage,
               step_all=np.array([e[0].elapsed_time(e[2]) for e in evs]),
               depth=to_numpy(r.depth), path=to_numpy(r.path), n_acc=to_numpy(r.n_acc))
    for _ in range(args.warmup):
        r.step(unfused=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        r.step(ev=evs[i], unfused=True)
    r.check()
    stage_u = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(4)] for e in evs])
    out["unfused_stage_ms"] = stage_u.mean(axis=0)
    out["unfused_step_all"] = np.array([e[0].elapsed_time(e[4]) for e in evs])
    if args.step_only:
        out["offset_paths"] = np.zeros((0, B, N), np.int32)
        out["offset_naccs"] = np.zeros((0, B), np.int32)
        return out

    def time_leg(call):
        """Per-call ms of `call` over `steps` launches, events on the launch stream."""
        for _ in range(args.warmup):
            call()
        evs_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e in evs_:
            e[0].record(stream)
            call()
            e[1].record(stream)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in evs_])

    # greedy verification (temperature 0) of the same batch, timed on its own
    g_path = torch.empty((B, N), dtype=torch.int32, device=dev)
    g_nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    g_toks = torch.empty((B, N), dtype=torch.int32, device=dev)
    ws_s, ws_s_n = r.ws_s, r.ws_s.numel()
    out["greedy_ms"] = time_leg(tav.prepare(
        "spec_verify_sample", d["target_logits"], None, d["parent"], d["token"], B, N, V, 0.0, 0,
        0, g_path, g_nacc, g_toks, ws_s, ws_s_n, flags, stream))
    out["greedy_nacc"] = to_numpy(g_nacc)

    # the walk under the without-replacement sibling rule (the trees' siblings
    # are distinct tokens), same inputs and uniforms as the step's
    out["wor_ms"] = time_leg(tav.prepare(
        "spec_verify_sample_wor", d["target_logits"], d["draft_logits"], d["parent"], d["token"],
        B, N, V, w.temperature, w.philox_seed, w.philox_offset, g_path, g_nacc, g_toks, ws_s,
        ws_s_n, flags, stream))
    out["wor_nacc"] = to_numpy(g_nacc)

    # the zero-copy rollback on the same paths, timed on its own: it moves
    # rows only inside each sequence's tree positions L..L+N-1, which the
    # attention never reads
    nblk, maxb = int(w.k_cache.shape[0]), int(w.block_table.shape[1])
    out["inplace_ms"] = time_leg(tav.prepare(
        "kv_commit_inplace", r.path, r.n_acc, nblk, d["block_table"], maxb, d["prefix_len"],
        r.copies[0][0], r.copies[0][1], B, N, w.Hkv, w.D, w.block, r.slots, r.new_len, flags,
        stream))

    # tree expansion over every node's draft row (top-4 tokens, log q,
    # entropy): one read of B*N vocabulary rows
    ex_rows = d["draft_logits"].view(B * N, V)
    ex_k = 4
    ex_tok = torch.empty((B * N, ex_k), dtype=torch.int32, device=dev)
    ex_lq = torch.empty((B * N, ex_k), dtype=torch.float64, device=dev)
    ex_ent = torch.empty((B * N,), dtype=torch.float64, device=dev)
    ex_ws = torch.empty(tav.tree_expand_workspace_bytes(B * N, V, ex_k), dtype=torch.uint8,
                        device=dev)
    out["expand_ms"] = time_leg(tav.prepare(
        "tree_expand_topk", ex_rows, B * N, V, ex_k, 1.0, ex_tok, ex_lq, ex_ent, ex_ws,
        ex_ws.numel(), flags, stream))
    out["expand_rows"] = B * N
    # the same rows with the k tokens drawn without replacement
    out["expand_sample_ms"] = time_leg(tav.prepare(
        "tree_expand_sample", ex_rows, B * N, V, ex_k, 1.0, w.philox_seed, w.philox_offset,
        ex_tok, ex_lq, ex_ent, ex_ws, ex_ws.numel(), flags, stream))

    # the budget step of tree construction: keep 64 of a 357-node candidate
    # tree per sequence (widths 4, 4, 3, 2, 2) by cumulative log q
    sel_widths, sel_M = (4, 4, 3, 2, 2), 64
    sel_par = [-1]
    sel_depth = [0]
    i = 0
    while i < len(sel_par):
        if sel_depth[i] < len(sel_widths):
            for _ in range(sel_widths[sel_depth[i]]):
                sel_par.append(i)
                sel_depth.append(sel_depth[i] + 1)
        i += 1
    Nc = len(sel_par)
    gen = torch.Generator(device="cpu").manual_seed(17)
    sel_parent = torch.tensor(sel_par, dtype=torch.int32).repeat(B, 1).to(dev)
    sel_token = torch.randint(0, V, (B, Nc), generator=gen, dtype=torch.int32).to(dev)
    sel_logq = torch.log(torch.rand((B, Nc), generator=gen, dtype=torch.float64)).to(dev)
    sel_out = [torch.empty((B, sel_M), dtype=torch.int32, device=dev) for _ in range(3)]
    out["select_ms"] = time_leg(tav.prepare(
        "tree_select_topm", sel_parent, sel_token, sel_logq, B, Nc, sel_M, *sel_out, flags,
        stream))
    out["select_shape"] = (B, Nc, sel_M)

    # the budget's best topology by dynamic programming (acceptance by sibling
    # rank, the rates read off the walk over Philox offsets below): timed here
    # for a 64-node, depth-6, width-4 budget with placeholder rates
    p_guess = [0.5, 0.25, 0.15, 0.1]
    topo = tav.tree_topology_dp(p_guess, 64, 6, device=dev)
    topo_need = int(tav.lib().tree_topology_workspace_bytes(4, 64, 6))
    topo_ws = torch.empty(max(topo_need, 1), dtype=torch.uint8, device=dev)
    import ctypes
    topo_p = (ctypes.c_double * 4)(*p_guess)
    out["topology_ms"] = time_leg(tav.prepare(
        "tree_topology_dp", ctypes.cast(topo_p, ctypes.c_void_p), 4, 64, 6, topo[0], topo[1],
        topo[2], topo_ws, topo_need, stream))

    # entropy-ranked widths (1..4) for a 64-node frontier per sequence
    wid_h = (torch.rand((B, 64), generator=gen, dtype=torch.float64) * 5).to(dev)
    wid_out = torch.empty((B, 64), dtype=torch.int32, device=dev)
    out["widths_ms"] = time_leg(tav.prepare("tree_widths_by_entropy", wid_h, B, 64, 1, 4, wid_out,
                                            flags, stream))

    # the speedup model's overhead per candidate position: the whole step at
    # tree sizes 1..N, each the first n nodes of the same best-first trees
    # (a best-first tree's first n nodes are its budget-n tree), timed alone
    sizes = [n for n in (1, 2, 4, 8, 16, 32, 64, 128, 256) if n <= N]
    size_us = []
    kc, vc = r.copies[0]
    for n in sizes:
        sl = {k: d[k][:, :n].contiguous() for k in ("parent", "token", "q", "k_tree", "v_tree",
                                                     "target_logits", "draft_logits")}
        m_n = torch.empty((B, n, (n + 63) // 64), dtype=torch.int64, device=dev)
        dep_n = torch.empty((B, n), dtype=torch.int32, device=dev)
        o_n = torch.empty((B, n, w.Hq, w.D), dtype=torch.float32, device=dev)
        wa = tav.new_attn_workspace(B, n, w.Hq, w.Hkv, w.D, w.max_prefix_len, dev)
        ws = tav.new_sampler_workspace(B, n, V, dev)
        pa = torch.empty((B, n), dtype=torch.int32, device=dev)
        na = torch.empty((B,), dtype=torch.int32, device=dev)
        tk = torch.empty((B, n), dtype=torch.int32, device=dev)
        sl_slots = torch.empty((B, n), dtype=torch.int32, device=dev)
        nl = torch.empty((B,), dtype=torch.int32, device=dev)
        seq = (
            tav.prepare("tree_attn_verify_tree", sl["q"], sl["k_tree"], sl["v_tree"], kc, vc,
                        nblk, d["block_table"], maxb, d["prefix_len"], w.max_prefix_len,
                        sl["parent"], m_n, dep_n, B, n, w.Hq, w.Hkv, w.D, w.block, w.scale, o_n,
                        wa, wa.numel(), flags, stream),
            tav.prepare("spec_verify_sample_commit", sl["target_logits"], sl["draft_logits"],
                        sl["parent"], sl["token"], B, n, V, w.temperature, w.philox_seed,
                        w.philox_offset, 0, pa, na, tk, sl["k_tree"], sl["v_tree"], nblk,
                        d["block_table"], maxb, d["prefix_len"], kc, vc, w.Hkv, w.D, w.block,
                        sl_slots, nl, ws, ws.numel(), flags, stream),
        )

        def step_n(seq=seq):
            for c in seq:
                c()
        size_us.append(float(np.median(time_leg(step_n))) * 1e3)
        del sl, m_n, dep_n, o_n, wa, ws
    out["size_n"] = sizes
    out["size_us"] = size_us

    # acceptance over many Philox offsets (outside the timed regions): the
    # mean accepted length and the rows the walk visits, for the byte count
    n_off = max(0, args.offsets)
    paths, naccs = r.offsets(n_off) if n_off else (np.zeros((0, B, N), np.int32),
                                                  np.zeros((0, B), np.int32))
    out["offset_paths"] = paths
    out["offset_naccs"] = naccs
    return out


def run_config(w, steps, warmup, n_offsets, flush, dev):
    """One workload's step timed cold: step and stage times, attention
    roofline, acceptance, and the step's roofline at the mean visited rows."""
    from synth.device import to_numpy

    r = StepRunner(w, dev, copies=1)
    r.ramp(0.1)
    step, stage = r.cold_steps(steps, warmup, flush)
    depth = to_numpy(r.depth)
    paths, naccs = r.offsets(n_offsets)
    acc = acceptance_stats(w, paths, naccs)
    a_bytes, a_flops = attention_work(w, depth)
    t_attn = float(np.median(stage[:, 0])) * 1e-3
    t_step = float(np.median(step)) * 1e-3
    floor = max((a_bytes + acc["mean_sampler_bytes"] + acc["mean_commit_bytes"]) / (HBM_PEAK_GBS * 1e9),
                a_flops / (MFMA_PEAK_TFLOPS * 1e12))
    res = {"workload": workload_desc(w), "step_us": round(t_step * 1e6, 2),
           "step_us_pctl": pct(step), "nodes_per_s": round(w.B * w.N / t_step, 1),
           "emitted_tokens_per_s": round(acc["mean_emitted_per_step"] / t_step, 1),
           "stages_us": {k: round(float(np.median(stage[:, i])) * 1e3, 2)
                         for i, k in enumerate(STAGES)},
           "tree_attn_roofline": roofline(a_bytes, a_flops, t_attn),
           "step_roofline": {"floor_us": round(floor * 1e6, 2), "frac": round(floor / t_step, 4)},
           "acceptance": acc}
    del r
    import torch
    torch.cuda.empty_cache()
    return res


def measured_copy_gbs(reps=5):
    """HBM rate of a plain 1 GiB device copy (read + write), timed with
    events: the streaming rate this machine reaches, beside the 8 TB/s figure."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.add(src, 0.0, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.add(src, 0.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / sec / 1e9


def copy_calibration(reps=5):
    """A plain device copy of COPY_BYTES (read and written once each), for
    scaling the HBM counters of the attention launch."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": reps}), flush=True)


def cpu_baseline(w, min_seconds=10.0, threads=None, sample=None):
    """The oracle's whole step (oracle.verify_step_ref) on the host, repeated
    for at least `min_seconds`, as verified tree nodes/s; `threads` caps the
    BLAS threads (None: all)."""
    import threadpoolctl

    import oracle
    with threadpoolctl.threadpool_limits(limits=threads):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.verify_step_ref(w)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
        info = threadpoolctl.threadpool_info()
        blas = max([i.get("num_threads", 1) for i in info] or [1])
    per_step = el / reps
    what = sample or f"the whole step ({w.B} sequences x {w.N} nodes)"
    return {"value": round(w.B * w.N / per_step, 2), "unit": "nodes/s", "cores": int(blas),
            "kind": "oracle",
            "sample": (f"{what} repeated {reps} times in {el:.1f} s; fp64 numpy attention on "
                       f"{blas} BLAS threads, single-threaded C walk; "
                       f"{len(os.sched_getaffinity(0))} cores visible")}


def sweep_model(sweep, decode, copy_gbs):
    """For each batch size and acceptance: the speedup model of a whole
    8B-shaped decoding step for the 16-node tree and the 6-node chain from
    their measured attention and walk times against a decode step's (the same
    workload cut to its root), the better of the two, and the best chain
    length for the chain's realised acceptance and overhead."""
    import tree_attention_verification_ancestor_amd as tav

    def times(rec):
        st = rec["stages_us"]
        return st["tree_attn_verify_tree"], st["spec_verify_sample_commit"]

    out = []
    for acc in SWEEP_ACCEPTS:
        for B in SWEEP_BATCHES:
            dec = decode[B]
            ad, sd = dec["stages_us"]["tree_attn_verify_tree"], \
                dec["stages_us"]["spec_verify_sample_commit"]
            row = {"B": B, "target_acceptance": acc}
            for rec in sweep:
                if rec["B"] != B or rec["target_acceptance"] != acc:
                    continue
                n = 16 if rec["tree"] == "tree16" else 6
                av, sv = times(rec)
                E = rec["acceptance"]["mean_emitted_per_step"] / B
                sp, alpha, td, tv = tav.verify_speedup(
                    E, 0.0, LAYERS_8B, LAYER_PARAMS_8B, HEAD_PARAMS_8B, B, n, av, sv, ad, sd,
                    copy_gbs, MFMA_PEAK_TFLOPS)
                row[rec["tree"]] = {"emitted_per_seq": round(E, 3), "speedup": round(sp, 3),
                                    "alpha": round(alpha, 4), "t_decode_us": round(td, 1),
                                    "t_verify_us": round(tv, 1)}
                if rec["tree"] == "chain6":
                    p = rec["acceptance"]["realised_acceptance"] or 0.0
                    nb, sb = tav.best_chain_length(p, 0.0, max(alpha, 0.0), 64)
                    row["best_chain"] = {"n": nb, "speedup": round(sb, 3), "acceptance": p}
            row["choice"] = max(("tree16", "chain6"), key=lambda k: row[k]["speedup"])
            out.append(row)
    return out


# The 32K-context config's trees, built on the GPU by the library's tree
# construction calls (treebuild.entropy_tree: the glossary's entropy-based
# branching and budget step): the root takes LONG_ROOT_WIDTH children, every
# later level gives each frontier node a width from its entropy rank in
# [LONG_W_MIN, LONG_W_MAX], for LONG_DEPTH levels over LONG_ROWS synthetic
# rows per sequence, and the budget step keeps the LONG_BUDGET best nodes by
# cumulative log q.
LONG_ROWS, LONG_DEPTH, LONG_ROOT_WIDTH, LONG_W_MIN, LONG_W_MAX, LONG_BUDGET = 256, 8, 4, 0, 3, 128


def run_configs(args, dev, copy_gbs):
    """The tiny, 8B, 70B TP-8 share, sweep and long-context workloads."""
    import torch

    from synth import make_workload
    from synth.workloads import slice_batch, slice_nodes, with_acceptance

    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    steps, warm, offs = args.config_steps, args.warmup, args.config_offsets
    cpu = not args.no_cpu
    res = {}

    def log(msg):
        print(f"[configs] {msg}", file=sys.stderr, flush=True)

    for name in ("tiny", "llama8b", "llama70b_tp8", "long"):
        tree_info = None
        if name == "long":
            from synth.workloads import gather_nodes
            big = make_workload(name, N=LONG_ROWS)
            import torch

            from synth.device import to_numpy
            from tree_attention_verification_ancestor_amd.treebuild import entropy_tree
            draft = torch.from_numpy(big.draft_logits).to(dev)
            op, ot, src, sizes = entropy_tree(draft, big.temperature, LONG_DEPTH,
                                              LONG_ROOT_WIDTH, LONG_W_MIN, LONG_W_MAX,
                                              LONG_BUDGET)
            w = gather_nodes(big, to_numpy(op), to_numpy(ot), to_numpy(src))
            del big, draft
            depth = np.zeros(w.N, np.int64)
            for i in range(1, w.N):
                depth[i] = depth[w.parent[0, i]] + 1
            tree_info = {"built_by": "tree_expand_topk + tree_widths_by_entropy + "
                                     "tree_select_topm on the GPU",
                         "candidate_level_sizes": sizes, "candidates": int(sum(sizes)),
                         "kept": int(w.N), "kept_depth_seq0": int(depth.max()),
                         "root_width": LONG_ROOT_WIDTH, "widths": [LONG_W_MIN, LONG_W_MAX]}
        else:
            w = make_workload(name)
        log(f"{name}: generated")
        rec = run_config(w, steps, warm, offs, flush, dev)
        if cpu:
            if name == "long":
                one = slice_batch(w, 1)
                rec["cpu_baseline"] = cpu_baseline(
                    one, min_seconds=3.0, sample="one sequence of the batch (128 nodes, 32K prefix)")
            else:
                rec["cpu_baseline"] = cpu_baseline(w, min_seconds=3.0)
                rec["cpu_baseline_1thread"] = cpu_baseline(w, min_seconds=2.0, threads=1)
        if tree_info:
            rec["tree"] = tree_info
        res[name] = rec
        log(f"{name}: step {rec['step_us']} us")
        del w

    sweep = []
    decode = {}
    for tname in ("sweep_tree16", "sweep_chain6"):
        base = make_workload(tname, B=max(SWEEP_BATCHES), accept=SWEEP_ACCEPTS[0],
                             keep_noise=True)
        log(f"{tname}: generated")
        for acc in SWEEP_ACCEPTS:
            wa = base if acc == SWEEP_ACCEPTS[0] else with_acceptance(base, acc)
            for B in SWEEP_BATCHES:
                w = slice_batch(wa, B)
                rec = run_config(w, steps, warm, offs, flush, dev)
                rec.update({"tree": tname.split("_")[1], "B": B, "target_acceptance": acc})
                if cpu and B == 1:
                    rec["cpu_baseline"] = cpu_baseline(w, min_seconds=1.0,
                                                       sample="the whole step at batch 1")
                    rec["cpu_baseline_1thread"] = cpu_baseline(
                        w, min_seconds=1.0, threads=1, sample="the whole step at batch 1")
                sweep.append(rec)
                log(f"{tname} accept {acc} B={B}: step {rec['step_us']} us, "
                    f"emitted/step {rec['acceptance']['mean_emitted_per_step']}")
                if tname == "sweep_chain6" and acc == 0.8:
                    # the decode step of this batch: the workload cut to its root
                    dec = run_config(slice_nodes(w, 1), steps, warm, offs, flush, dev)
                    decode[B] = dec
                    log(f"decode B={B}: step {dec['step_us']} us")
            del wa
        del base
    res["sweep"] = sweep
    res["sweep_decode"] = [{"B": B, "step_us": decode[B]["step_us"],
                            "stages_us": decode[B]["stages_us"]} for B in SWEEP_BATCHES]
    res["sweep_model"] = sweep_model(sweep, decode, copy_gbs)
    del flush
    torch.cuda.empty_cache()
    return res


def speedup_model(sizes, size_us):
    """The pages' speedup model fed by this GPU's step times: alpha from the
    times at tree sizes 1..N, then the best chain length and its model
    speedup at acceptance 0.8 and 0.9 with no draft cost."""
    import tree_attention_verification_ancestor_amd as tav

    alpha = tav.fit_alpha(sizes, size_us)
    rec = {"n": sizes, "step_us": [round(t, 2) for t in size_us], "alpha": round(alpha, 5),
           "ceiling": round(1.0 / alpha, 2) if alpha > 0 else None, "best_chain": {}}
    for p in (0.8, 0.9):
        n, s = tav.best_chain_length(p, 0.0, alpha, 1024)
        rec["best_chain"][str(p)] = {"n": n, "speedup": round(s, 3)}
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama70b")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    ap.add_argument("--accept", type=float, default=None,
                    help="mean acceptance of a sweep workload (0.5, 0.8 or 0.9)")
    ap.add_argument("--cache-copies", type=int, default=3)
    ap.add_argument("--offsets", type=int, default=1000,
                    help="Philox offsets of the acceptance statistics run")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (no tiny/8B/TP-8 share/sweep/long)")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps per config")
    ap.add_argument("--config-offsets", type=int, default=100,
                    help="Philox offsets of each config's acceptance run")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone: no timed legs for the other calls, no "
                         "tree-size sweep and no configs (for counter passes)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain copy of known size (for the HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU: no collectives or sharding across GPUs are built)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    from synth import make_workload
    from tree_attention_verification_ancestor_amd.profiling import current_traffic
    over = {}
    if args.batch is not None:
        over["B"] = args.batch
    if args.accept is not None:
        over["accept"] = args.accept
    w = make_workload(args.config, **over)
    g = run_headline(args, w)
    copy_gbs = measured_copy_gbs()

    attn_bytes, attn_flops = attention_work(w, g["depth"])
    t_attn = g["ms_attn"] * 1e-3
    tflops = attn_flops / t_attn / 1e12
    gbs = attn_bytes / t_attn / 1e9
    t_hbm = attn_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = attn_flops / (MFMA_PEAK_TFLOPS * 1e12)
    traffic = current_traffic(TRAFFIC_RECORD) if args.config == "llama70b" and not over else None
    roof = roofline(attn_bytes, attn_flops, t_attn)
    roof["traffic"] = traffic

    step_bytes = attn_bytes + sampler_bytes(w, g["path"], g["n_acc"]) + commit_bytes(w, g["n_acc"])
    offp, offn = g["offset_paths"], g["offset_naccs"]
    acceptance = None
    if len(offn) > 0:
        acceptance = acceptance_stats(w, offp, offn)
        acceptance["step_floor_us_at_mean"] = round(max(
            (attn_bytes + acceptance["mean_sampler_bytes"] + acceptance["mean_commit_bytes"])
            / (HBM_PEAK_GBS * 1e9), t_mfma) * 1e6, 2)
    topology = None
    if len(offn) > 0 and "topology_ms" in g:
        import tree_attention_verification_ancestor_amd as tav
        rates, tried = rank_acceptance(w, offp, offn, K=4)
        parent, rank, value = tav.tree_topology_dp(rates, w.N, 6)
        parent = parent.cpu().numpy()
        depth = np.zeros(w.N, np.int64)
        for i in range(1, w.N):
            depth[i] = depth[parent[i]] + 1
        topology = {"rank_acceptance": [round(r, 4) for r in rates],
                    "rank_tries": [int(t) for t in tried],
                    "n": w.N, "depth_limit": 6,
                    "expected_accepted": round(float(value.cpu().numpy()[0]), 4),
                    "nodes_per_depth": np.bincount(depth).tolist(),
                    "best_first_tree_mean_accepted": acceptance["mean_accepted_per_seq"],
                    "us": pct(g["topology_ms"])}
    t_floor = max(step_bytes / (HBM_PEAK_GBS * 1e9), t_mfma)
    ms = g["ms_step"]
    rec = {
        "metric": "verified tree nodes/s",
        "value": round(w.B * w.N / (ms * 1e-3), 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload_desc(w), "global_batch": w.B, "tree_nodes": w.N,
                   "prefix_tokens": int(w.prefix_len.sum()), "vocab": w.V,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "verify_step_us": round(ms * 1e3, 2),
        "stages_us": {k: round(v * 1e3, 2) for k, v in zip(STAGES, g["stage_ms"])},
        "stages_us_pctl": {k: pct(g["stage_all"][:, i]) for i, k in enumerate(STAGES)},
        "step_us_pctl": pct(g["step_all"]),
        "unfused_step": {"us_pctl": pct(g["unfused_step_all"]),
                         "stages_us": {k: round(v * 1e3, 2)
                                       for k, v in zip(STAGES_UNFUSED, g["unfused_stage_ms"])}},
        "tree_attn": {"us": round(t_attn * 1e6, 2), "us_pctl": pct(g["attn_all"]),
                      "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "measured_copy_gbs": round(copy_gbs, 1),
                      "hbm_frac_of_copy": round(gbs / copy_gbs, 4),
                      "tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                      "algorithmic_bytes": attn_bytes, "algorithmic_flops": attn_flops,
                      "roofline_frac": round(max(t_hbm, t_mfma) / t_attn, 4)},
        "step_roofline": {"algorithmic_bytes": step_bytes, "floor_us": round(t_floor * 1e6, 2),
                          "frac": round(t_floor / (ms * 1e-3), 4)},
        "accepted": g["n_acc"].tolist(),
        "acceptance": acceptance,
    }
    if "greedy_ms" in g:
        rec.update({
            "greedy": {"spec_verify_sample_us": pct(g["greedy_ms"]),
                       "accepted": g["greedy_nacc"].tolist()},
            "without_replacement": {"spec_verify_sample_wor_us": pct(g["wor_ms"]),
                                    "accepted": g["wor_nacc"].tolist()},
            "kv_commit_inplace_us": pct(g["inplace_ms"]),
            "speedup_model": speedup_model(g["size_n"], g["size_us"]),
            "tree_widths_by_entropy": {"B": w.B, "F": 64, "us": pct(g["widths_ms"])},
            "tree_topology_dp": topology,
            "tree_expand_sample": {"rows": g["expand_rows"], "k": 4, "us": pct(g["expand_sample_ms"])},
            "tree_select_topm": {"B": g["select_shape"][0], "Nc": g["select_shape"][1],
                                 "M": g["select_shape"][2], "us": pct(g["select_ms"])},
            "tree_expand_topk": {"rows": g["expand_rows"], "k": 4, "us": pct(g["expand_ms"]),
                                 "hbm_gbs": round(g["expand_rows"] * w.V * 4
                                                  / (float(np.median(g["expand_ms"])) * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(g["expand_rows"] * w.V * 4
                                                   / (float(np.median(g["expand_ms"])) * 1e-3)
                                                   / (HBM_PEAK_GBS * 1e9), 4)},
        })
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w)
    del w, g
    torch.cuda.empty_cache()
    if not (args.no_configs or args.step_only):
        rec["configs"] = run_configs(args, torch.device("cuda:0"), copy_gbs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
