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

  python -m top_selection_row_amd.profiling collect --workload W --raw DIR \
        --out profiles [--tag T] [-- extra bench.py arguments]
      runs every pass on a GPU host, each a child process: the kernel trace,
      FETCH_SIZE and WRITE_SIZE of bench.py and of its 512 MiB copy, and two
      passes of SQ counters (instruction mix, VALU and LDS activity, waits, LDS
      bank and address conflicts); writes deepselect_<tag>_trace.txt,
      deepselect_<tag>_traffic.json and deepselect_<tag>_sq.txt to --out.

  python -m top_selection_row_amd.profiling table --out FILE [--workloads ...]
      runs bench.py once per workload (library choices, torch.topk beside it)
      and writes the table of per-call time, throughput, fraction of the HBM
      peak and W against its bound.
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


SQ_PASSES = [
    ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
     "SQ_ACTIVE_INST_VALU", "SQ_THREAD_CYCLES_VALU"],
    ["SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
     "SQ_LDS_ADDR_CONFLICT", "SQ_INSTS_LDS_ATOMIC", "SQ_ACTIVE_INST_SCA"],
]


def sq_derived(cs: dict) -> dict:
    """Ratios of one kernel's SQ counters (each a sum over waves and instances)."""
    out = {}
    waves = cs.get("SQ_WAVES", 0.0)
    wc = cs.get("SQ_WAVE_CYCLES", 0.0)
    if waves:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_LDS_ATOMIC"):
            if c in cs:
                out[f"{c[3:].lower()}_per_wave"] = cs[c] / waves
    if wc:
        for c, name in (("SQ_ACTIVE_INST_VALU", "valu_active_share"), ("SQ_ACTIVE_INST_LDS", "lds_active_share"),
                        ("SQ_ACTIVE_INST_SCA", "salu_active_share"), ("SQ_WAIT_ANY", "wait_any_share"),
                        ("SQ_WAIT_INST_ANY", "wait_inst_any_share"), ("SQ_WAIT_INST_LDS", "wait_inst_lds_share")):
            if c in cs:
                out[name] = cs[c] / wc
    if cs.get("SQ_ACTIVE_INST_VALU"):
        # active lanes per VALU instruction cycle, over 64
        out["valu_lane_utilisation"] = cs.get("SQ_THREAD_CYCLES_VALU", 0.0) / (64.0 * cs["SQ_ACTIVE_INST_VALU"])
    if cs.get("SQ_ACTIVE_INST_LDS"):
        out["lds_bank_conflict_per_active_cycle"] = cs.get("SQ_LDS_BANK_CONFLICT", 0.0) / cs["SQ_ACTIVE_INST_LDS"]
        out["lds_addr_conflict_per_active_cycle"] = cs.get("SQ_LDS_ADDR_CONFLICT", 0.0) / cs["SQ_ACTIVE_INST_LDS"]
    return out


def _run(cmd, log, timeout):
    import subprocess

    log.append(" ".join(cmd))
    print("[collect] " + " ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"), timeout=timeout,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        print(res.stdout[-3000:], flush=True)
        raise RuntimeError(f"step failed ({res.returncode}): {' '.join(cmd)}")
    return res.stdout


def cmd_collect(a):
    bench = os.path.join(ROOT, "bench.py")
    raw = os.path.abspath(a.raw)
    out = os.path.abspath(a.out)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    tag = a.tag or a.workload
    extra = list(a.extra or [])
    py = sys.executable
    bargs = [py, bench, "--workload", a.workload, "--no-cpu-baseline", "--no-torch"] + extra
    prof = ["rocprofv3"]
    cmds = []
    # 1. kernel trace
    _run(prof + ["--kernel-trace", "--stats", "--output-format", "csv", "-d", f"{raw}/trace", "-o", "trace", "--"]
         + bargs + ["--steps", str(a.steps), "--warmup", "20"], cmds, 300)
    tr = argparse.Namespace(dir=f"{raw}/trace", title=f"DeepSelect {tag}: rocprofv3 kernel trace",
                            cmd=f"python -m top_selection_row_amd.profiling collect {' '.join(sys.argv[2:])} "
                                f"(pass: {cmds[-1]})", match="deepselect")
    import contextlib
    import io

    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        cmd_trace(tr)
    with open(os.path.join(out, f"deepselect_{tag}_trace.txt"), "w") as f:
        f.write(buf.getvalue())
    # 2. traffic: FETCH_SIZE and WRITE_SIZE of the call and of a known copy
    dirs = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        for what, args in (("kernel", bargs + ["--steps", "50", "--warmup", "5"]),
                           ("copy", [py, bench, "--mode", "copy", "--copy-mb", "512", "--steps", "20", "--warmup", "3"])):
            d = f"{raw}/pmc_{ctr}_{what}"
            _run(prof + ["--pmc", ctr, "--output-format", "csv", "-d", d, "-o", "pmc", "--"] + args, cmds, 180)
            dirs[(ctr, what)] = d
    tf = argparse.Namespace(workload=a.workload, kernel_fetch=dirs[("FETCH_SIZE", "kernel")],
                            kernel_write=dirs[("WRITE_SIZE", "kernel")], copy_fetch=dirs[("FETCH_SIZE", "copy")],
                            copy_write=dirs[("WRITE_SIZE", "copy")], copy_bytes=512.0 * 2**20,
                            cmd=[f"python -m top_selection_row_amd.profiling collect {' '.join(sys.argv[2:])}"]
                            + cmds[-4:], out=os.path.join(out, f"deepselect_{tag}_traffic.json"))
    with contextlib.redirect_stdout(io.StringIO()):
        cmd_traffic(tf)
    # 3. SQ counters, two passes
    merged = defaultdict(dict)
    for i, ctrs in enumerate(SQ_PASSES):
        d = f"{raw}/sq{i}"
        _run(prof + ["--pmc"] + ctrs + ["--output-format", "csv", "-d", d, "-o", "pmc", "--"]
             + bargs + ["--steps", "20", "--warmup", "5"], cmds, 180)
        for k, cs in counters(d, "deepselect").items():
            merged[k].update(cs)
    lines = [f"# DeepSelect {tag}: SQ counters per dispatch (summed over the kernel's waves and instances)",
             f"# command: python -m top_selection_row_amd.profiling collect {' '.join(sys.argv[2:])}"]
    lines += [f"#   pass: {c}" for c in cmds[-2:]]
    for k, cs in merged.items():
        lines.append(f"== {k}")
        for c, v in sorted(cs.items()):
            lines.append(f"   {c:34s} {v:16.1f}")
        for c, v in sq_derived(cs).items():
            lines.append(f"   {c:34s} {v:16.4f}")
    with open(os.path.join(out, f"deepselect_{tag}_sq.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def cmd_table(a):
    bench = os.path.join(ROOT, "bench.py")
    rows = []
    for wl in a.workloads:
        cmd = [sys.executable, bench, "--workload", wl, "--no-cpu-baseline", "--steps", str(a.steps),
               "--warmup", "20"]
        txt = _run(cmd, [], 300)
        line = [l for l in txt.splitlines() if l.startswith("{")][-1]
        rows.append(json.loads(line))
    out = ["# DeepSelect on one MI355X, every workload (library choice of split and waves)",
           f"# command: python -m top_selection_row_amd.profiling table {' '.join(sys.argv[2:])}",
           "# (each row: python3 bench.py --workload W --no-cpu-baseline; per-call time = K calls back to back",
           "# between two HIP events on the launch stream; torch.topk on the same rotating buffers)", "",
           "| workload | batch x N, dtype | k | split | us per call | Gelem/s | GB/s | frac of 8 TB/s "
           "| torch.topk us (unsorted / sorted) | W mean / bound (max / bound) |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for d in rows:
        c, w, t = d["config"], d["w_stats"], d.get("torch_topk") or {}
        out.append(f"| {c['workload']} | {c['batch']} x {c['N']} {c['input_dtype']} | {c['k']} | {c['split']} "
                   f"| {d['kernel_us']['avg']:.2f} | {d['value']:.1f} | {d['roofline']['achieved']:.0f} "
                   f"| {d['roofline']['frac']:.4f} | {t.get('unsorted_us', '-')} / {t.get('sorted_us', '-')} "
                   f"| {w['mean_over_bound']:.3f} ({w['max_over_bound']:.3f}) |")
    text = "\n".join(out) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text, flush=True)


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
    co = sub.add_parser("collect")
    co.add_argument("--workload", required=True)
    co.add_argument("--raw", required=True, help="directory for rocprofv3's raw output")
    co.add_argument("--out", required=True, help="directory for the summaries")
    co.add_argument("--tag", default="")
    co.add_argument("--steps", type=int, default=200)
    co.add_argument("extra", nargs="*", help="more bench.py arguments (after --)")
    co.set_defaults(fn=cmd_collect)
    tb = sub.add_parser("table")
    tb.add_argument("--out", required=True)
    tb.add_argument("--steps", type=int, default=200)
    tb.add_argument("--workloads", nargs="*", default=["gauss4k", "dsa32k", "dsa128k_bf16", "vocab152k_k64",
                                                       "vocab152k_k1024", "asc1m", "ties1m", "asc1m_b1"])
    tb.set_defaults(fn=cmd_table)
    a = ap.parse_args(argv)
    a.fn(a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
