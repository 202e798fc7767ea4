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
    for k in ATTN_KERNELS:
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
        "# HBM traffic of one tree_attn_verify launch (main kernel + combine), from",
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", required=True, help="the commands that made the runs, ' ;; '-separated")
    a = ap.parse_args()
    rec = write_record(a.out, counter_means(a.fetch), counter_means(a.write), counter_means(a.copy_fetch),
                       counter_means(a.copy_write), a.copy_bytes, a.command)
    print(rec)


if __name__ == "__main__":
    main()
