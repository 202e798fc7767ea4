"""rocprofv3 summaries: per-kernel counter means and the HBM traffic record.

The HBM traffic of the attention launch comes from two counter passes over
the benchmark (FETCH_SIZE, then WRITE_SIZE, each in KiB per dispatch). Both
counters are scaled by what they read for a plain device-to-device copy of
known size, so the figure is in bytes of HBM traffic. The record names the
SHA-256 of the kernel source it was taken from; a reader that finds a
different source treats the figure as stale.

    python -m tree_attention_verification_ancestor_amd.profiling \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --copy-bytes N --out profiles/FILE.txt --command "..."
    python -m tree_attention_verification_ancestor_amd.profiling \\
        --counters DIR [DIR ...] --out profiles/FILE.txt --command "..."

The second form writes per-kernel counter means over several counter passes
(each pass within the hardware's per-block counter limits) and the ratios
derived from them.

    python -m tree_attention_verification_ancestor_amd.profiling \
        --trace DIR --title "..." --out profiles/FILE.md --command "..."

The third form writes a kernel-trace summary: dispatches and durations per
kernel and grid, with the SHA-256 of every library source.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCE = os.path.join(PKG, "csrc", "tree_attn.hip")
ATTN_KERNELS = ("tree_attn_kernel", "tree_attn_combine_kernel")


def source_sha256(path: str = ATTN_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_means(run_dir: str) -> dict:
    """{kernel short name: {counter: mean value per dispatch}} from the
    counter_collection CSV(s) under a rocprofv3 output directory."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    sums = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    for path in files:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                name = short_name(r["Kernel_Name"])
                sums[name][r["Counter_Name"]] += float(r["Counter_Value"])
                disp[name].add((path, r["Dispatch_Id"]))
    return {k: {c: v / len(disp[k]) for c, v in cs.items()} for k, cs in sums.items()}


def short_name(kernel: str) -> str:
    for k in ATTN_KERNELS + ("spec_verify_kernel",):
        if k in kernel:
            return k
    if "FunctorOnSelf_add" in kernel:     # torch.add(src, 0, out=dst): the calibration copy
        return "copy"
    return kernel.split("(")[0][-80:]


def write_record(out: str, fetch: dict, write: dict, copy_fetch: dict, copy_write: dict,
                 copy_bytes: int, command: str) -> dict:
    cf = copy_fetch["copy"]["FETCH_SIZE"] * 1024.0 / copy_bytes
    cw = copy_write["copy"]["WRITE_SIZE"] * 1024.0 / copy_bytes
    lines = [
        "# HBM traffic of one attention launch (the main kernel, and the combine kernel",
        "# when more than two splits are merged; tree_attn_verify and",
        "# tree_attn_verify_tree run the same kernels), from",
        "# rocprofv3 counter passes; KiB per dispatch as the counters read them, then",
        "# bytes after dividing by the copy-kernel factors (counter bytes per true byte).",
        "# commands (from the repository root):",
    ] + [f"#   {c}" for c in command.split(" ;; ")] + [
        f"kernel_source_sha256 = {source_sha256()}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {copy_fetch['copy']['FETCH_SIZE']:.1f}",
        f"copy_write_kib = {copy_write['copy']['WRITE_SIZE']:.1f}",
        f"fetch_factor = {cf:.4f}",
        f"write_factor = {cw:.4f}",
    ]
    total = 0.0
    for k in ATTN_KERNELS:
        if k not in fetch and k not in write:
            continue   # not launched in this workload (the combine kernel at two splits)
        fk = fetch.get(k, {}).get("FETCH_SIZE", 0.0)
        wk = write.get(k, {}).get("WRITE_SIZE", 0.0)
        b = fk * 1024.0 / cf + wk * 1024.0 / cw
        total += b
        lines += [f"{k}.fetch_kib = {fk:.1f}", f"{k}.write_kib = {wk:.1f}", f"{k}.hbm_bytes = {b:.0f}"]
    lines.append(f"traffic_bytes_per_launch = {total:.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return read_record(out)


def read_record(path: str) -> dict:
    rec = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or "=" not in line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            rec[k] = v
    return rec


def current_traffic(path: str):
    """Bytes per attention launch from the record at `path`, or None when the
    record is missing or was taken from a different kernel source."""
    if not os.path.exists(path):
        return None
    rec = read_record(path)
    if rec.get("kernel_source_sha256") != source_sha256():
        return None
    return int(float(rec["traffic_bytes_per_launch"]))


MOPS_FLOPS = 512   # FLOPs per unit of the SQ_INSTS_VALU_MFMA_MOPS_* counters


def trace_rows(run_dir: str) -> list:
    """[(kernel, grid, workgroup, [durations us])] from the kernel_trace CSV(s)
    under a rocprofv3 output directory, in order of first dispatch."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {run_dir}")
    rows = {}
    for path in files:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                name = name[5:] if name.startswith("void ") else name
                name = name.replace("tav::(anonymous namespace)::", "").split("(")[0]
                wg = int(r.get("Workgroup_Size", r.get("Workgroup_Size_X", 0)) or 0)
                grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
                key = (name, grid // max(wg, 1), wg)
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                rows.setdefault(key, []).append(dur)
    return [(k[0], k[1], k[2], v) for k, v in rows.items()]


def write_trace_summary(out: str, run_dir: str, title: str, command: str, note: str = "") -> list:
    """Markdown table of a kernel trace: per library kernel and grid, the
    dispatch count and mean / min / max duration; the other kernels (torch's
    fills and copies) summed in one line."""
    rows = trace_rows(run_dir)
    ours = [r for r in rows if not r[0].startswith(("at::", "__amd", "void at::"))]
    other = [d for r in rows if r not in ours for d in r[3]]
    total = sum(sum(r[3]) for r in rows)
    lines = [f"# {title}", ""] + ([note, ""] if note else []) + [
        "Command (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):", ""]
    lines += [f"    {c}" for c in command.split(" ;; ")]
    lines += ["", "| kernel | workgroups × threads | dispatches | mean µs | min µs | max µs | share of kernel time |",
              "|---|---|---|---|---|---|---|"]
    for name, wgs, wg, d in sorted(ours, key=lambda r: -sum(r[3])):
        lines.append(f"| {name} | {wgs} × {wg} | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | "
                     f"{max(d):.2f} | {100 * sum(d) / total:.1f} % |")
    if other:
        lines.append(f"| (torch fills and copies, all) | | {len(other)} | {sum(other) / len(other):.2f} | "
                     f"{min(other):.2f} | {max(other):.2f} | {100 * sum(other) / total:.1f} % |")
    lines += ["", "Library sources at the time of the trace (SHA-256):", ""]
    for path in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        lines.append(f"- {os.path.basename(path)} {source_sha256(path)}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return ours


def derived_counters(c: dict, xcds: int, simds: int) -> dict:
    """Ratios from one kernel's counter means (each formula is in its key):
    the MFMA pipes' busy share of SIMD-cycles (GRBM_GUI_ACTIVE is summed over
    the XCDs), wave-cycles spent waiting, LDS bank conflicts per LDS-active
    cycle, and the MFMA FLOPs the op counters imply."""
    d = {}
    gui = c.get("GRBM_GUI_ACTIVE")
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        d["mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / xcds * simds)"] = \
            c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / xcds * simds)
    if c.get("SQ_WAVE_CYCLES"):
        for k in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY"):
            if k in c:
                d[f"{k} / SQ_WAVE_CYCLES"] = c[k] / c["SQ_WAVE_CYCLES"]
    if c.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in c:
        d["SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
    mops = sum(v for k, v in c.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    if mops:
        d[f"mfma_flops = sum(SQ_INSTS_VALU_MFMA_MOPS_*) * {MOPS_FLOPS}"] = mops * MOPS_FLOPS
    return d


def write_counter_summary(out: str, runs: list, kernels: list, xcds: int, simds: int,
                          command: str) -> dict:
    """Per-kernel counter means (per dispatch) over several counter passes,
    with the derived ratios; returns {kernel: {name: value}}."""
    merged = defaultdict(dict)
    for run in runs:
        for k, cs in run.items():
            merged[k].update(cs)
    lines = ["# rocprofv3 counter means per dispatch, by kernel, with derived ratios",
             "# commands (from the repository root):"] + [f"#   {c}" for c in command.split(" ;; ")] + [
             f"kernel_source_sha256 = {source_sha256()}", f"xcds = {xcds}", f"simds = {simds}"]
    result = {}
    for k in kernels:
        if k not in merged:
            continue
        c = dict(sorted(merged[k].items()))
        c.update(derived_counters(merged[k], xcds, simds))
        result[k] = c
        lines.append(f"[{k}]")
        lines += [f"{n} = {v:.6g}" for n, v in c.items()]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", required=True, help="the commands that made the runs, ' ;; '-separated")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=int)
    ap.add_argument("--counters", nargs="+", help="counter-pass directories: write a counter summary")
    ap.add_argument("--trace", help="a kernel-trace directory: write a trace summary")
    ap.add_argument("--title", default="Kernel trace")
    ap.add_argument("--note", default="", help="a paragraph under the title (the workload)")
    ap.add_argument("--kernels", nargs="+", default=list(ATTN_KERNELS) + ["spec_verify_kernel"])
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--simds", type=int, default=1024)
    a = ap.parse_args()
    if a.trace:
        for r in write_trace_summary(a.out, a.trace, a.title, a.command, a.note):
            print(r[0], r[1], r[2], len(r[3]), round(sum(r[3]) / len(r[3]), 2))
        return
    if a.counters:
        print(write_counter_summary(a.out, [counter_means(d) for d in a.counters], a.kernels, a.xcds,
                                    a.simds, a.command))
        return
    if not (a.fetch and a.write and a.copy_fetch and a.copy_write and a.copy_bytes):
        ap.error("the traffic record needs --fetch, --write, --copy-fetch, --copy-write, --copy-bytes")
    rec = write_record(a.out, counter_means(a.fetch), counter_means(a.write), counter_means(a.copy_fetch),
                       counter_means(a.copy_write), a.copy_bytes, a.command)
    print(rec)


if __name__ == "__main__":
    main()
