"""Benchmark of the tree-verification step on one MI355X.

A step is one pass of the whole path over one batch: tree_mask_build,
tree_attn_verify (one attention layer), spec_verify_sample and kv_commit_path,
chained on one stream with no host synchronisation. The workload is the
Llama-3-70B-shaped layer: batch 8, 64-node trees (depth 6, width 4), 64 query
/ 8 KV heads, head_dim 128, paged prefixes of 6144..8192 tokens, a 128256-entry
vocabulary. Inputs are seeded synthetic data already resident in HBM; three
copies of the paged caches rotate across steps so the 256 MB last-level cache
cannot hold the step's KV working set.

Prints one JSON line: verified tree nodes/s (B*N per step time), with the
attention launch's roofline and the CPU oracle's rate on this host; per-stage
and per-step percentiles from a second pass with events between the calls;
and, outside the timed regions, the walk's acceptance over many Philox
offsets (mean accepted length, emitted tokens, rows visited). The
attention launch (main kernel + combine) is timed with events on its stream
inside the timed region; its HBM traffic comes from the rocprofv3 counter
record under profiles/ while that record matches the kernel source.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config llama70b] [--no-cpu]
                    [--offsets 1000]
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


def run_gpu(args, w):
    import torch

    import tree_attention_verification_ancestor_amd as tav
    from synth.device import to_numpy, upload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = upload(w, dev)
    copies = [(d["k_cache"], d["v_cache"])]
    for _ in range(args.cache_copies - 1):
        copies.append((d["k_cache"].clone(), d["v_cache"].clone()))
    B, N, V = w.B, w.N, w.V
    flags = tav.new_flags(dev)
    mask = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    out = torch.empty((B, N, w.Hq, w.D), dtype=torch.float32, device=dev)
    ws_a = torch.empty(max(1, tav.tree_attn_workspace_bytes(B, N, w.Hq, w.Hkv, w.D,
                                                            w.max_prefix_len)),
                       dtype=torch.uint8, device=dev)
    ws_s = tav.new_sampler_workspace(B, N, V, dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
    toks = torch.empty((B, N), dtype=torch.int32, device=dev)
    slots = torch.empty((B, N), dtype=torch.int32, device=dev)
    new_len = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    nblk, maxb = int(w.k_cache.shape[0]), int(w.block_table.shape[1])
    ws_a_n = ws_a.numel()
    ws_s_n = ws_s.numel()

    # one checked call of each entry point, then pre-marshalled calls for the loop
    tav.tree_mask_build(d["parent"], mask, depth, flags, stream)
    tav.tree_attn_verify(d["q"], d["k_tree"], d["v_tree"], copies[0][0], copies[0][1],
                         d["block_table"], d["prefix_len"], w.max_prefix_len, mask, w.scale, out,
                         ws_a, flags, stream)
    tav.spec_verify_sample(d["target_logits"], d["draft_logits"], d["parent"], d["token"],
                           w.temperature, w.philox_seed, w.philox_offset, path, n_acc, toks, ws_s,
                           flags, stream)
    tav.kv_commit_path(d["k_tree"], d["v_tree"], path, n_acc, d["block_table"], d["prefix_len"],
                       copies[0][0], copies[0][1], slots, new_len, flags, stream)
    torch.cuda.synchronize()
    calls = []
    for kc, vc in copies:
        calls.append((
            tav.prepare("tree_mask_build", d["parent"], B, N, mask, depth, flags, stream),
            tav.prepare("tree_attn_verify", d["q"], d["k_tree"], d["v_tree"], kc, vc, nblk,
                        d["block_table"], maxb, d["prefix_len"], w.max_prefix_len, mask, B, N,
                        w.Hq, w.Hkv, w.D, w.block, w.scale, out, ws_a, ws_a_n, flags, stream),
            tav.prepare("spec_verify_sample", d["target_logits"], d["draft_logits"], d["parent"],
                        d["token"], B, N, V, w.temperature, w.philox_seed, w.philox_offset, path,
                        n_acc, toks, ws_s, ws_s_n, flags, stream),
            tav.prepare("kv_commit_path", d["k_tree"], d["v_tree"], path, n_acc, nblk,
                        d["block_table"], maxb, d["prefix_len"], kc, vc, B, N, w.Hkv, w.D,
                        w.block, slots, new_len, flags, stream),
        ))

    def step(i, ev=None, attn_ev=None):
        c = calls[i % len(calls)]
        if ev:
            ev[0].record(stream)
        for k in range(4):
            if attn_ev and k == 1:
                attn_ev[0].record(stream)
            c[k]()
            if attn_ev and k == 1:
                attn_ev[1].record(stream)
            if ev:
                ev[k + 1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps between two synchronised events;
    # the attention launch of every step is bracketed by events on its stream
    attn_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, attn_ev=attn_evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    ms_attn = float(np.mean([e[0].elapsed_time(e[1]) for e in attn_evs]))

    # per-stage times with events on the launch stream (a second pass)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    stage = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(4)] for e in evs])
    stage_ms = stage.mean(axis=0)
    step_ms = np.array([e[0].elapsed_time(e[4]) for e in evs])
    assert int(flags.item()) == 0, f"device flags {int(flags.item()):#x}"
    out = dict(ms_step=ms_step, ms_attn=ms_attn, stage_ms=stage_ms, stage_all=stage,
               step_all=step_ms, depth=to_numpy(depth), path=to_numpy(path), n_acc=to_numpy(n_acc))

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
    out["inplace_ms"] = time_leg(tav.prepare(
        "kv_commit_inplace", path, n_acc, nblk, d["block_table"], maxb, d["prefix_len"],
        copies[0][0], copies[0][1], B, N, w.Hkv, w.D, w.block, slots, new_len, flags, stream))

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
    for n in sizes:
        sl = {k: d[k][:, :n].contiguous() for k in ("parent", "token", "q", "k_tree", "v_tree",
                                                     "target_logits", "draft_logits")}
        m_n = torch.empty((B, n, (n + 63) // 64), dtype=torch.int64, device=dev)
        dep_n = torch.empty((B, n), dtype=torch.int32, device=dev)
        o_n = torch.empty((B, n, w.Hq, w.D), dtype=torch.float32, device=dev)
        wa = torch.empty(max(1, tav.tree_attn_workspace_bytes(B, n, w.Hq, w.Hkv, w.D,
                                                              w.max_prefix_len)),
                         dtype=torch.uint8, device=dev)
        ws = tav.new_sampler_workspace(B, n, V, dev)
        pa = torch.empty((B, n), dtype=torch.int32, device=dev)
        na = torch.empty((B,), dtype=torch.int32, device=dev)
        tk = torch.empty((B, n), dtype=torch.int32, device=dev)
        sl_slots = torch.empty((B, n), dtype=torch.int32, device=dev)
        nl = torch.empty((B,), dtype=torch.int32, device=dev)
        kc, vc = copies[0]
        seq = (
            tav.prepare("tree_mask_build", sl["parent"], B, n, m_n, dep_n, flags, stream),
            tav.prepare("tree_attn_verify", sl["q"], sl["k_tree"], sl["v_tree"], kc, vc, nblk,
                        d["block_table"], maxb, d["prefix_len"], w.max_prefix_len, m_n, B, n,
                        w.Hq, w.Hkv, w.D, w.block, w.scale, o_n, wa, wa.numel(), flags, stream),
            tav.prepare("spec_verify_sample", sl["target_logits"], sl["draft_logits"],
                        sl["parent"], sl["token"], B, n, V, w.temperature, w.philox_seed,
                        w.philox_offset, pa, na, tk, ws, ws.numel(), flags, stream),
            tav.prepare("kv_commit_path", sl["k_tree"], sl["v_tree"], pa, na, nblk,
                        d["block_table"], maxb, d["prefix_len"], kc, vc, B, n, w.Hkv, w.D,
                        w.block, sl_slots, nl, flags, stream),
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
    paths = torch.empty((n_off, B, N), dtype=torch.int32, device=dev)
    naccs = torch.empty((n_off, B), dtype=torch.int32, device=dev)
    toks_o = torch.empty((n_off, B, N), dtype=torch.int32, device=dev)
    for o in range(n_off):
        tav.spec_verify_sample(d["target_logits"], d["draft_logits"], d["parent"], d["token"],
                               w.temperature, w.philox_seed, o, paths[o], naccs[o], toks_o[o],
                               ws_s, flags, stream)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0, f"device flags {int(flags.item()):#x}"
    out["offset_paths"] = to_numpy(paths)
    out["offset_naccs"] = to_numpy(naccs)
    return out


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


def cpu_baseline(w, min_seconds=10.0):
    import threadpoolctl

    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.verify_step_ref(w)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per_step = el / reps
    info = threadpoolctl.threadpool_info()
    blas = max([i.get("num_threads", 1) for i in info] or [1])
    return {"value": w.B * w.N / per_step, "unit": "nodes/s", "cores": int(blas),
            "kind": "oracle",
            "sample": (f"the whole step ({w.B} sequences x {w.N} nodes) repeated {reps} times in "
                       f"{el:.1f} s; fp64 numpy attention on {blas} BLAS threads, "
                       f"single-threaded C walk; {len(os.sched_getaffinity(0))} cores visible")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama70b")
    ap.add_argument("--cache-copies", type=int, default=3)
    ap.add_argument("--offsets", type=int, default=1000,
                    help="Philox offsets of the acceptance statistics run")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone: no timed legs for the other calls and no "
                         "tree-size sweep (for counter passes)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain copy of known size (for the HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; see DESIGN.md for how it would shard)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    from synth import make_workload
    from tree_attention_verification_ancestor_amd.profiling import current_traffic
    w = make_workload(args.config)
    g = run_gpu(args, w)
    copy_gbs = measured_copy_gbs()

    attn_bytes, attn_flops = attention_work(w, g["depth"])
    t_attn = g["ms_attn"] * 1e-3
    tflops = attn_flops / t_attn / 1e12
    gbs = attn_bytes / t_attn / 1e9
    t_hbm = attn_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = attn_flops / (MFMA_PEAK_TFLOPS * 1e12)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    traffic = current_traffic(TRAFFIC_RECORD) if args.config == "llama70b" else None
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}

    step_bytes = attn_bytes + sampler_bytes(w, g["path"], g["n_acc"]) + commit_bytes(w, g["n_acc"])
    pct = lambda a: {"p10": round(float(np.percentile(a, 10)) * 1e3, 2),
                     "p50": round(float(np.percentile(a, 50)) * 1e3, 2),
                     "p90": round(float(np.percentile(a, 90)) * 1e3, 2)}
    offp, offn = g["offset_paths"], g["offset_naccs"]
    acceptance = None
    if len(offn) > 0:
        samp_mean = float(np.mean([sampler_bytes(w, offp[o], offn[o]) for o in range(len(offn))]))
        acceptance = {
            "offsets": int(len(offn)),
            "mean_accepted_per_seq": round(float(offn.mean()), 4),
            "mean_emitted_per_step": round(float((offn + 1).sum(axis=1).mean()), 3),
            "mean_sampler_bytes": round(samp_mean),
            "step_floor_us_at_mean": round(max((attn_bytes + samp_mean + float(np.mean(
                [commit_bytes(w, offn[o]) for o in range(len(offn))]))) / (HBM_PEAK_GBS * 1e9),
                attn_flops / (MFMA_PEAK_TFLOPS * 1e12)) * 1e6, 2),
        }
    t_floor = max(step_bytes / (HBM_PEAK_GBS * 1e9), attn_flops / (MFMA_PEAK_TFLOPS * 1e12))
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
        "stages_us": {k: round(v * 1e3, 2) for k, v in
                      zip(["tree_mask_build", "tree_attn_verify", "spec_verify_sample",
                           "kv_commit_path"], g["stage_ms"])},
        "stages_us_pctl": {k: pct(g["stage_all"][:, i]) for i, k in
                           enumerate(["tree_mask_build", "tree_attn_verify",
                                      "spec_verify_sample", "kv_commit_path"])},
        "step_us_pctl": pct(g["step_all"]),
        "tree_attn": {"us": round(t_attn * 1e6, 2),
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
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
