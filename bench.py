#!/usr/bin/env python3
"""Benchmark of DeepSelect batched row-wise top-k on one MI355X.

One step = one deepselect_topk call over a whole batch (every block of every row
streamed once, filtered, compacted, and the k results written). The default
workload is the long-context DSA indexer case: 128 rows x 131072 bfloat16 scores
(causal -inf tails), k = 2048, B = B2 = 2048.

Timing
  * inputs are resident in HBM: R rotating copies of the batch (R*size >= the
    --rotate-mb budget, default 768 MiB, three times the 256 MiB Infinity Cache)
    so every launch reads rows that are not cached;
  * W untimed warm-up steps, then exactly K steps back to back, bracketed by a
    device synchronisation and a HIP event on the launch stream on both sides;
    the region time / K is the call's average duration, used for both the
    value and the roofline (no event between the calls: each costs the stream
    about 2 us of its own);
  * a separate pass brackets each of up to 100 more calls with its own pair
    of events, for their spread (kernel_us.event_pair_median);
  * value = batch*N / (region time / K) in Gelem/s (whole job, one GPU).

Extras in the JSON line: the roofline of the kernel (HBM-bound; algorithmic
bytes = input read once + k (value, index) pairs per row), the CPU oracle timed
on this host, and torch.topk on the same buffers.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "top-k Gelem/s and HBM GB/s (% of peak), batch×N rows, k=512/2048"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"deepselect_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    from top_selection_row_amd.profiling import source_digest

    if d.get("source_digest") != source_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(workload: str, seconds: float):
    import numpy as np

    import oracle
    import synth

    w = synth.WORKLOADS[workload]
    threads = max(1, min(16, os.cpu_count() or 1))
    rows = min(w.batch, 64)
    x = synth.generate(workload, rows)
    oracle.topk(x[:1], w.k, nthreads=1)  # load + warm
    done, t0 = 0, time.perf_counter()
    while True:
        oracle.topk(x, w.k, nthreads=threads)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gelem = done * rows * w.n / el / 1e9
    # the same oracle on one thread, over 8 rows for a third of the time
    rows1 = min(rows, 8)
    done1, t0 = 0, time.perf_counter()
    while True:
        oracle.topk(x[:rows1], w.k, nthreads=1)
        done1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= seconds / 3:
            break
    del np
    return {"value": round(gelem, 4), "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} passes of the oracle (C full sort) over {rows} of the {w.batch} "
                      f"rows, {el:.1f} s",
            "one_thread": round(done1 * rows1 * w.n / el1 / 1e9, 4),
            "host": f"{host_cpu()}, {os.cpu_count()} logical CPUs"}


def w_bound_row(n: int, k: int, B: int, B2: int, split: int = 1) -> float:
    """Expected total RadixSelectTopK input of a row, (1 + k/B2)(k + B + B2) H_m
    with m = ceil(N/B) (the DeepSelect deep-dive's boxed bound, section
    "RadixSelectTopK 总处理元素数的期望上界"), summed over a split row's parts
    (each with its own block count) and its merge (S blocks of k results)."""
    def one(n_, blk):
        m = -(-n_ // blk)
        return (1.0 + k / B2) * (k + blk + B2) * math.fsum(1.0 / i for i in range(1, m + 1))

    if split <= 1:
        return one(n, B)
    m = -(-n // B)
    parts = [min((s + 1) * m // split * B, n) - s * m // split * B for s in range(split)]
    return math.fsum(one(p, B) for p in parts) + one(split * k, k)


def w_stats(st, n, k, B, B2, split) -> dict:
    """Device W per row (parts and merge summed) against the bound."""
    W = st[:, 0].astype(float)
    bound = w_bound_row(n, k, B, B2, split)
    return {"rows": int(len(W)), "split": int(split), "W_mean": round(float(W.mean()), 1),
            "W_max": int(W.max()), "bound": round(bound, 1), "mean_over_bound": round(float(W.mean()) / bound, 4),
            "max_over_bound": round(float(W.max()) / bound, 4),
            "A_mean": round(float(st[:, 1].mean()), 1), "R_mean": round(float(st[:, 2].mean()), 2)}


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def copy_calibration(args, torch) -> int:
    """A plain copy of known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it
    gives the factor from those counters to bytes actually moved."""
    n = args.copy_mb * 2**20 // 4
    src = torch.randint(0, 1 << 30, (n,), dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": n * 4, "bytes_written": n * 4, "steps": args.steps,
                      "ms_per_copy": round(ms, 5), "GBps_read_plus_write": round(2 * n * 4 / ms / 1e6, 1)}),
          flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="dsa128k_bf16")
    ap.add_argument("--split", type=int, default=0, help="parts per row (0 = library choice)")
    ap.add_argument("--waves", type=int, default=0, help="waves per workgroup (0 = library choice)")
    ap.add_argument("--kernel", type=int, default=0,
                    help="0 library choice, 1 ring streaming, 2 register streaming, 3 generic")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sorted", action="store_true",
                    help="results of each row in descending order (ds_options_t.sorted)")
    ap.add_argument("--sample", action="store_true",
                    help="fused softmax and one draw per row (sorted output; ds_options_t.probs/sample_u)")
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--top-p", type=float, default=1.0)
    ap.add_argument("--share", action="store_true",
                    help="split rows share their parts' thresholds (ds_options_t.share_threshold)")
    ap.add_argument("--lengths", action="store_true",
                    help="pass each row's valid length (ds_options_t.lengths; causal rows end where their "
                         "-inf tail starts, other workloads are full rows)")
    ap.add_argument("--rotate-mb", type=int, default=768)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-torch", action="store_true", help="skip the torch.topk comparison")
    ap.add_argument("--mode", choices=("topk", "copy"), default="topk",
                    help="copy: time a plain device-to-device copy of --copy-mb MiB (the counter "
                         "calibration run for FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--copy-mb", type=int, default=512)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the DeepSelect path here has no multi-GPU leg "
              "(rows shard across GPUs without communication). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.mode == "copy":
        return copy_calibration(args, torch)

    import synth
    import top_selection_row_amd as ds

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    dt = ds.DS_F32 if w.dtype == "f32" else ds.DS_BF16
    es = w.elem_bytes

    log(f"[bench] generating {args.workload}: {w.batch} x {w.n} {w.dtype}")
    x = synth.generate(args.workload)
    size = x.nbytes
    copies = max(2, math.ceil(args.rotate_mb * 2**20 / size))
    if w.dtype == "f32":
        xt = torch.from_numpy(x).to(dev)
    else:
        xt = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    rot = torch.empty((copies, w.batch, w.n), dtype=xt.dtype, device=dev)
    for i in range(copies):
        rot[i].copy_(xt)
    del xt
    vals = torch.empty((w.batch, w.k), dtype=rot.dtype, device=dev)
    idx = torch.empty((w.batch, w.k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    split = args.split or ds.deepselect_plan_split(dt, w.batch, w.n, w.k, w.block, w.block2,
                                                   props.multi_processor_count)
    if split < 1:
        log(f"[bench] no valid split: {ds.deepselect_status_string(split)}")
        return 1
    lib = ds.library()
    lens = torch.from_numpy(synth.valid_lengths(args.workload)).to(dev) if args.lengths else None
    if args.sample:
        args.sorted = True
        probs = torch.empty((w.batch, w.k), dtype=torch.float32, device=dev)
        draws = torch.rand(w.batch, generator=torch.Generator().manual_seed(args.seed)).to(dev)
        sampled = torch.empty(w.batch, dtype=torch.int32, device=dev)
    opt = ds.DsOptions(int(split), int(args.waves), None, None, 0, int(args.kernel), int(args.sorted),
                       lens.data_ptr() if lens is not None else None,
                       probs.data_ptr() if args.sample else None, float(args.temperature), float(args.top_p),
                       draws.data_ptr() if args.sample else None, sampled.data_ptr() if args.sample else None,
                       int(args.share))
    ptrs = [rot[i].data_ptr() for i in range(copies)]
    vptr, iptr = vals.data_ptr(), idx.data_ptr()
    fn = lib.deepselect_topk_ex
    seed = args.seed

    def step(i):
        rc = fn(ptrs[i % copies], dt, w.batch, w.n, w.n, w.k, w.block, w.block2, seed, vptr, iptr, sptr,
                ctypes.byref(opt))
        if rc != 0:
            raise RuntimeError(f"deepselect_topk_ex failed: {ds.deepselect_status_string(rc)}")

    log(f"[bench] {copies} rotating copies ({copies * size / 2**20:.0f} MiB), split {split}, "
        f"{args.warmup} warm-up + {args.steps} timed steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # the timed region: K calls back to back, with events only at its ends (an
    # event recorded between calls costs the stream about 2 us of its own)
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = r0.elapsed_time(r1)
    ms_per_step = region_ms / K
    # the call's average duration on its stream over the timed region
    call_ms = ms_per_step
    # a separate pass of per-call event pairs, for their spread
    P = min(K, 100)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(P)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(P)]
    for i in range(P):
        ev0[i].record(stream)
        step(args.warmup + K + i)
        ev1[i].record(stream)
    torch.cuda.synchronize()
    pair_ms = sorted(a.elapsed_time(b) for a, b in zip(ev0, ev1))
    elems = w.batch * w.n
    value = elems / (ms_per_step * 1e-3) / 1e9
    # bytes the call must move: every (valid) input element once, and the output
    read_elems = int(lens.sum().item()) if lens is not None else w.batch * w.n
    alg_bytes = read_elems * es + w.batch * w.k * (es + 4)
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    log(f"[bench] region {region_ms:.3f} ms for {K} steps (wall {wall * 1e3:.1f} ms): {call_ms * 1e3:.2f} us per "
        f"call, {achieved:.0f} GB/s; per-call event pairs: median {pair_ms[P // 2] * 1e3:.2f} us")

    # one more call, untimed, with the device statistics: W against the bound
    st_dev = torch.empty((w.batch, 4), dtype=torch.int64, device=dev)
    opt_st = ds.DsOptions(int(split), int(args.waves), st_dev.data_ptr(), None, 0, int(args.kernel),
                          int(args.sorted), lens.data_ptr() if lens is not None else None, None, 1.0, 1.0, None,
                          None, int(args.share))
    rc = fn(ptrs[0], dt, w.batch, w.n, w.n, w.k, w.block, w.block2, seed, vptr, iptr, sptr, ctypes.byref(opt_st))
    if rc != 0:
        raise RuntimeError(f"deepselect_topk_ex failed: {ds.deepselect_status_string(rc)}")
    torch.cuda.synchronize()
    wst = w_stats(st_dev.cpu().numpy(), w.n, w.k, w.block, w.block2, split)
    if args.lengths:
        wst["note"] = "rows run on their valid prefixes; the bound is for full rows"
    log(f"[bench] W per row: mean {wst['W_mean']}, max {wst['W_max']}, bound {wst['bound']} "
        f"(mean/bound {wst['mean_over_bound']})")

    torch_info = None
    if not args.no_torch:
        tk = {}
        for srt in (False, True):
            for i in range(3):
                torch.topk(rot[i % copies], w.k, dim=-1, largest=True, sorted=srt)
            torch.cuda.synchronize()
            reps = min(50, K)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps):
                torch.topk(rot[i % copies], w.k, dim=-1, largest=True, sorted=srt)
            b.record(stream)
            torch.cuda.synchronize()
            tk["sorted_us" if srt else "unsorted_us"] = round(a.elapsed_time(b) / reps * 1e3, 2)
        torch_info = tk
        log(f"[bench] torch.topk: {tk}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu}")

    # the committed counter figures are for the plain call
    traffic = None if (args.sorted or args.lengths or args.sample or args.share) else measured_traffic(args.workload)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16" if w.dtype == "bf16" else "u32",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": w.batch, "N": w.n, "input_dtype": w.dtype,
                   "k": w.k, "B": w.block, "B2": w.block2, "split": int(split), "sorted": bool(args.sorted),
                   "lengths": bool(args.lengths), "share_threshold": bool(args.share),
                   "sample": ({"temperature": args.temperature, "top_p": args.top_p} if args.sample else None),
                   "rotating_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "kernel_us": {"avg": round(call_ms * 1e3, 3),
                      "event_pair_median": round(pair_ms[P // 2] * 1e3, 3), "event_pairs": P},
        "cpu_baseline": cpu,
        "torch_topk": torch_info,
        "w_stats": wst,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
