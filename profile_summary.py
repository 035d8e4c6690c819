"""Summarise rocprofv3 output of a bench.py run into profiles/.

  kernel stats:  rocprofv3 --kernel-trace --stats -d DIR -o run --output-format csv -- python3 bench.py ...
  counters:      rocprofv3 --pmc FETCH_SIZE -d DIR ... ; rocprofv3 --pmc WRITE_SIZE -d DIR ...
                 (bench.py --with-copy adds a 4 GiB copy kernel that calibrates both counters)

python3 profile_summary.py --name NAME --stats DIR [--fetch DIR --write DIR --kernel KEY=SUBSTR ...]
writes profiles/NAME.md (per-kernel average durations, counter bytes per
dispatch, the calibration factors and the commands) and, for every
--kernel KEY=SUBSTR, records HBM bytes per launch in profiles/traffic.json,
keyed by KEY and tied to the sha of the kernel's source file.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))
PROF = os.path.join(ROOT, "profiles")
COPY_BYTES = 32768 * 65536 * 2         # bench.py copy_calibration(): 4 GiB each way
SOURCES = {"grouped_gemm": "gemm.hip", "router": "router.hip", "dispatch": "dispatch.hip",
           "permute": "dispatch.hip", "quant": "quant.hip", "combine": "combine.hip", "bias": "combine.hip"}


def short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0][:80]


def find(d, pattern):
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[0]


def kernel_stats(d):
    rows = list(csv.DictReader(open(find(d, "*kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append((short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    return out


def counter(d, cname):
    rows = list(csv.DictReader(open(find(d, "*counter_collection.csv"))))
    per = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == cname:
            per[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


def sha(src):
    with open(os.path.join(ROOT, "sigmoid_top_routing_02_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--kernel", action="append", default=[], help="KEY=substring of the kernel name")
    ap.add_argument("--command", action="append", default=[], help="command lines to record")
    ap.add_argument("--note", default="")
    ap.add_argument("--step", action="append", default=[],
                    help="substring of a kernel that belongs to the benchmark's timed step; with any given, "
                         "the other kernels of the process (input generation, weight preparation, the copy "
                         "calibration, error checks) are listed in a table of their own")
    a = ap.parse_args()
    lines = [f"# {a.name}", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["Commands (run from the repository root on an MI355X):", ""]
    lines += [f"    {c}" for c in a.command] + [""]
    stats = sorted(kernel_stats(a.stats), key=lambda x: -x[3])
    in_step = [r for r in stats if not a.step or any(sub in r[0] for sub in a.step)]
    other = [r for r in stats if a.step and not any(sub in r[0] for sub in a.step)]
    head = ["| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    lines += ["## Kernel durations (rocprofv3 --kernel-trace --stats)", ""]
    if a.step:
        lines += ["Kernels of the timed step (calls include the warm-up steps):", ""]
    lines += head
    for n, c, avg, tot, pct in in_step:
        lines.append(f"| {n} | {c} | {avg:.1f} | {tot:.2f} | {pct:.1f} |")
    if other:
        lines += ["", "Other kernels of the same process, outside the timed step (input and weight "
                  "generation, offline weight quantisation, the copy calibration and copy ceiling, "
                  "error checks):", ""] + head
        for n, c, avg, tot, pct in other:
            lines.append(f"| {n} | {c} | {avg:.1f} | {tot:.2f} | {pct:.1f} |")
    if a.fetch and a.write:
        fetch, write = counter(a.fetch, "FETCH_SIZE"), counter(a.write, "WRITE_SIZE")
        copy_key = next(k for k in fetch if "permute_rows" in k)
        # the copy kernel runs first: its first two dispatches are the calibration
        f_copy = min(fetch[copy_key][:2]) * 1024.0
        w_copy = min(write[copy_key][:2]) * 1024.0
        f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
        lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)", "",
                  f"Copy calibration: 4 GiB copy kernel read {f_copy / 2**20:.1f} MiB (FETCH_SIZE) and wrote "
                  f"{w_copy / 2**20:.1f} MiB (WRITE_SIZE): scale factors {f_scale:.4f} and {w_scale:.4f}.", "",
                  "| kernel | dispatches | FETCH MiB/dispatch | WRITE MiB/dispatch | scaled GB/dispatch |",
                  "|---|---|---|---|---|"]
        tj_path = os.path.join(PROF, "traffic.json")
        tj = json.load(open(tj_path)) if os.path.exists(tj_path) else {}
        for k in sorted(fetch):
            fv = fetch[k][2:] if k == copy_key else fetch[k]
            wv = write.get(k, [0.0])[2:] if k == copy_key else write.get(k, [0.0])
            if not fv:
                continue
            fm = sum(fv) / len(fv) * 1024.0
            wm = sum(wv) / max(len(wv), 1) * 1024.0
            tot = fm * f_scale + wm * w_scale
            lines.append(f"| {k} | {len(fv)} | {fm / 2**20:.1f} | {wm / 2**20:.1f} | {tot / 1e9:.3f} |")
            for spec in a.kernel:
                key, sub = spec.split("=", 1)
                if sub in k:
                    src = next((v for s, v in SOURCES.items() if s in k), None)
                    tj[key] = {"kernel": k, "bytes_per_launch": round(tot), "fetch_bytes": round(fm * f_scale),
                               "write_bytes": round(wm * w_scale), "source_sha": sha(src) if src else None,
                               "profile": f"profiles/{a.name}.md"}
        json.dump(tj, open(tj_path, "w"), indent=1, sort_keys=True)
    open(os.path.join(PROF, f"{a.name}.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
