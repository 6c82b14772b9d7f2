"""Summaries of rocprofv3 output for the MoE decode kernels.

    python -m quantized_expert_gemv_amd.profiling stats  <run_kernel_stats.csv>
    python -m quantized_expert_gemv_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> --copy-bytes N --workload NAME --out profiles/traffic_NAME.json

`traffic` turns the per-dispatch FETCH_SIZE / WRITE_SIZE counters (KiB) of
each kernel into bytes per launch, each counter scaled by what it reads for
a plain device copy of N bytes run in the same process (the benchmark runs it
last: the process's last copyBuffer dispatch; weight uploads and slot copies
come before it), and records the digest of the kernel sources the
counters were taken with, so a later benchmark can tell whether they still
describe the current kernels.
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))


def _code_only(text: str) -> str:
    """The source without its comments and blank lines (string literals in
    these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln)


def src_digest() -> str:
    """Digest of the kernel and host sources as code: an edit of comments
    alone leaves it unchanged."""
    h = hashlib.sha256()
    for f in ("layer.hip", "b1_layer.hip", "b8_layer.hip", "dense.hip", "prefill.hip", "kernel_common.h",
              "device_util.h", "api.cpp", "moe_internal.h"):
        with open(os.path.join(_PKG, "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """Demangled kernel name without return type, argument list and anonymous namespace."""
    k = kernel.replace("(anonymous namespace)::", "")
    k = k.split("(")[0]
    return k.replace("void ", "").strip()


def kernel_stats(path: str) -> list[dict]:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def counter_means(path: str) -> dict:
    agg = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            agg[(short_name(r["Kernel_Name"]), r["Counter_Name"])].append(float(r["Counter_Value"]))
    return agg


def last_copy(path: str, counter: str) -> float:
    """The counter of the last copyBuffer dispatch (highest dispatch id)."""
    best = None
    with open(path) as f:
        for r in csv.DictReader(f):
            if short_name(r["Kernel_Name"]) == "__amd_rocclr_copyBuffer" and r["Counter_Name"] == counter:
                d = int(r["Dispatch_Id"])
                if best is None or d > best[0]:
                    best = (d, float(r["Counter_Value"]))
    if best is None:
        raise SystemExit(f"no copyBuffer dispatch in {path}")
    return best[1]


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int) -> dict:
    fetch, write = counter_means(fetch_csv), counter_means(write_csv)
    copy_f = last_copy(fetch_csv, "FETCH_SIZE")
    copy_w = last_copy(write_csv, "WRITE_SIZE")
    kf = copy_bytes / (copy_f * 1024.0)
    kw = copy_bytes / (copy_w * 1024.0)
    out = {"copy_bytes": copy_bytes, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
           "fetch_factor": kf, "write_factor": kw, "kernels": {}}
    for (name, cnt), vals in fetch.items():
        if not name.startswith("moe::"):
            continue
        w = write.get((name, "WRITE_SIZE"), [0.0])
        fk, wk = sum(vals) / len(vals), sum(w) / len(w)
        out["kernels"][name] = {"dispatches": len(vals), "fetch_kib": fk, "write_kib": wk,
                                "bytes_per_launch": fk * 1024 * kf + wk * 1024 * kw}
    return out


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--dominant", default="k_fused_layer")
    t.add_argument("--out")
    a = p.parse_args()
    if a.cmd == "stats":
        print("| kernel | calls | avg us | min us | max us | % time |\n|---|---|---|---|---|---|")
        for r in kernel_stats(a.csv):
            print(f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                  f"{r['max_us']:.2f} | {r['pct']:.1f} |")
    else:
        t = traffic(a.fetch_csv, a.write_csv, a.copy_bytes)
        dom = next((v for k, v in t["kernels"].items() if a.dominant in k), None)
        t.update({"workload": a.workload, "src_digest": src_digest(),
                  "dominant_kernel": a.dominant,
                  "dominant_bytes_per_launch": None if dom is None else dom["bytes_per_launch"]})
        text = json.dumps(t, indent=1, sort_keys=True)
        if a.out:
            with open(a.out, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    main()
