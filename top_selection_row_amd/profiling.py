"""Summaries of rocprofv3 output for the DeepSelect kernels.

Used to turn rocprofv3 runs of ``bench.py`` into the short text summaries kept
under ``profiles/`` (and the HBM-traffic figure ``bench.py`` reports). It reads
only rocprofv3's CSV output; nothing here touches a GPU.

Commands (each summary records the full command lines that produced it):

  python -m top_selection_row_amd.profiling trace DIR [--title T] [--cmd C]
      kernel-trace statistics (rocprofv3 --kernel-trace --stats
      --output-format csv): calls, total, average, min, max per kernel.

  python -m top_selection_row_amd.profiling counters DIR [--match NAME]
      per-dispatch averages of every counter in a --pmc run (summed over the
      counter's hardware instances).

  python -m top_selection_row_amd.profiling traffic --workload W \
        --kernel-fetch DIR --kernel-write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes N [--out FILE]
      HBM bytes per call (the DeepSelect kernels of one call summed) from
      FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for
      a plain copy kernel of known size (bytes read = bytes written = N per
      copy).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_digest() -> str:
    """Digest of the kernel sources (a traffic figure is valid only for them)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_selection_row_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def short(name: str) -> str:
    name = name.split("(")[0]
    return name.replace("void ", "")


def trace_stats(d: str):
    """Rows of rocprofv3's kernel_stats.csv (times in ns)."""
    rows = []
    with open(_find(d, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append(r)
    return rows


def kernel_durations(d: str, match: str):
    """Per-dispatch durations (ns) of kernels whose name contains `match`."""
    out = []
    with open(_find(d, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if match in r["Kernel_Name"]:
                out.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def counters(d: str, match: str = "deepselect"):
    """{kernel: {counter: mean over dispatches of the value summed over instances}}."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    with open(_find(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if match not in name:
                continue
            per[short(name)][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    out = {}
    for k, cs in per.items():
        out[k] = {c: statistics.fmean(v.values()) for c, v in cs.items()}
    return out


def cmd_trace(a):
    rows = trace_stats(a.dir)
    print(f"# {a.title or 'rocprofv3 kernel trace'}")
    if a.cmd:
        print(f"# command: {a.cmd}")
    print(f"{'kernel':70s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
    for r in rows:
        print(f"{short(r['Name'])[:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
              f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    if a.match:
        # a call runs the part kernel once, plus the merge kernel when rows are
        # split: the per-call time is the matching kernels' total over the calls
        per = [(short(r["Name"]), float(r["TotalDurationNs"]) / 1e3, int(r["Calls"]))
               for r in rows if a.match in r["Name"]]
        if per:
            calls = max(c for _, _, c in per)
            total = sum(t for _, t, _ in per) / calls
            print(f"# per call ({' + '.join(n.split('<')[0].split('::')[-1] for n, _, _ in per)}, "
                  f"{calls} calls): {total:.2f} us (total duration / calls)")


def cmd_counters(a):
    res = counters(a.dir, a.match)
    if a.cmd:
        print(f"# command: {a.cmd}")
    for k, cs in res.items():
        print(f"== {k}")
        for c, v in sorted(cs.items()):
            print(f"   {c:32s} {v:16.1f}")


def cmd_traffic(a):
    kf = counters(a.kernel_fetch, "deepselect")
    kw = counters(a.kernel_write, "deepselect")
    cf = counters(a.copy_fetch, "copyBuffer")
    cw = counters(a.copy_write, "copyBuffer")

    def pick(d, c):
        vals = [cs[c] for cs in d.values() if c in cs]
        if not vals:
            raise KeyError(f"counter {c} missing")
        return vals

    # FETCH_SIZE / WRITE_SIZE are reported in KiB per dispatch
    copy_fetch = max(pick(cf, "FETCH_SIZE")) * 1024.0
    copy_write = max(pick(cw, "WRITE_SIZE")) * 1024.0
    f_scale = a.copy_bytes / copy_fetch
    w_scale = a.copy_bytes / copy_write
    kern = {}
    for k, cs in kf.items():
        if "FETCH_SIZE" in cs:
            kern.setdefault(k, {})["fetch_bytes"] = cs["FETCH_SIZE"] * 1024.0 * f_scale
    for k, cs in kw.items():
        if "WRITE_SIZE" in cs:
            kern.setdefault(k, {})["write_bytes"] = cs["WRITE_SIZE"] * 1024.0 * w_scale
    # a call launches each DeepSelect kernel once: per-call bytes are the sum
    fetch = sum(v.get("fetch_bytes", 0.0) for v in kern.values())
    write = sum(v.get("write_bytes", 0.0) for v in kern.values())
    out = {
        "workload": a.workload,
        "source_digest": source_digest(),
        "kernels": sorted(kern),
        "fetch_bytes_per_launch": fetch,
        "write_bytes_per_launch": write,
        "hbm_bytes_per_launch": fetch + write,
        "copy_calibration": {"copy_bytes": a.copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale},
        "all_kernels": kern,
        "commands": a.cmd,
    }
    text = json.dumps(out, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", default="")
    t.add_argument("--cmd", default="")
    t.add_argument("--match", default="deepselect")
    t.set_defaults(fn=cmd_trace)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--match", default="deepselect")
    c.add_argument("--cmd", default="")
    c.set_defaults(fn=cmd_counters)
    r = sub.add_parser("traffic")
    r.add_argument("--workload", required=True)
    r.add_argument("--kernel-fetch", required=True)
    r.add_argument("--kernel-write", required=True)
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--copy-bytes", type=float, required=True)
    r.add_argument("--cmd", default="", nargs="*")
    r.add_argument("--out", default="")
    r.set_defaults(fn=cmd_traffic)
    a = ap.parse_args(argv)
    a.fn(a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
