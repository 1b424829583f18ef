"""Throughput of batched nucleus sampling on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]

A step is one nucleus_sample call over one batch: validate, max, min-p,
top-k, top-p cut, renormalise and the exponential race for every row.  The
default workload is B = 256 rows of V = 128256 fp32 Zipf-shaped logits
(workloads.py, workload 3).  Inputs sit in HBM before timing starts; the
timed steps rotate over enough copies of the batch (> 512 MB in total) that
the 256 MB last-level cache cannot serve a repeat read.

Prints one JSON line: rows/s for the whole job, the dominant kernel's
achieved HBM bandwidth against the 8 TB/s peak (per-launch HIP events on the
stream the kernel runs on), the same buffers read by a pure streaming kernel
for comparison, the same calls writing the probabilities out, the other
workloads (small, ties, chain in bf16, flat) timed the same way, the
rejection sampler, speculative verification and the pre-chain on the
benchmark batch, and the float64 oracle timed on the host's cores over a
bounded sample of the same rows.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "sampled rows/sec and logits HBM GB/s (% of peak) at B=256, V=128256 fp32"
# Every source of the library: a change to any of them invalidates committed counters.
KERNEL_SOURCES = sorted(os.path.relpath(p, ROOT) for p in glob.glob(
    os.path.join(ROOT, "nucleus_sampling_amd", "csrc", "*")) if p.endswith((".h", ".hip")))


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        p = os.path.join(ROOT, rel)
        if os.path.exists(p):
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name: str, bytes_per_launch: float):
    """HBM bytes per launch from committed rocprofv3 PMC counters, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("traffic_bytes_per_launch")


CAL_BYTES = 256 * 2**20  # bytes read and written by the calibration kernel


def _pmc_rows(d: str):
    """(kernel name, counter value) per dispatch from a rocprofv3 counter_collection CSV under d."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((r.get("Kernel_Name", ""), float(r.get("Counter_Value", "nan"))))
    return rows


def pmc_summary(fetch_dir: str, write_dir: str, name: str, shape, dtype: str):
    """Per-launch HBM bytes of the sampler's kernels from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the calibration kernel (CAL_BYTES read and written)."""
    import numpy as np
    B, V = shape
    algo = B * V * (2 if dtype == "bf16" else 4)
    out = {"workload": name, "kernel_hash": kernel_hash(), "algorithmic_bytes_per_launch": algo,
           "calibration": f"torch.add over {CAL_BYTES} bytes (reads and writes CAL_BYTES)"}
    per = {}
    for label, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _pmc_rows(d)
        cal = [v for k, v in rows if "elementwise" in k and "add" in k.lower() and "Fill" not in k]
        if not cal:
            raise SystemExit(f"no calibration dispatch found under {d}")
        factor = CAL_BYTES / (np.median(cal) * 1024.0)
        kern = {}
        for k, v in rows:
            for short in ("row_kernel", "race_kernel", "probs_kernel", "tile_kernel"):
                if f"nucleus::{short}" in k or k.startswith(short) or f" {short}<" in k or f"{short}<" in k:
                    kern.setdefault(short, []).append(v)
        per[label] = {"scale_factor": factor, "calibration_counter_kib": float(np.median(cal)),
                      "kernels": {k: {"dispatches": len(v), "counter_kib_mean": float(np.mean(v)),
                                      "bytes_per_dispatch": float(np.mean(v)) * 1024.0 * factor}
                                  for k, v in kern.items()}}
    out.update(per)
    fetch = sum(v["bytes_per_dispatch"] for v in per["fetch"]["kernels"].values())
    write = sum(v["bytes_per_dispatch"] for v in per["write"]["kernels"].values())
    out["traffic_bytes_per_launch"] = fetch + write
    out["fetch_over_algorithmic"] = fetch / algo
    path = os.path.join(ROOT, "profiles", f"pmc_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def host_cpus():
    """What the host offers and what the oracle may use: the machine's CPU share
    for one GPU is OMP_NUM_THREADS (16 there), whatever os.cpu_count() shows."""
    logical = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = logical
    try:
        import psutil
        physical = psutil.cpu_count(logical=False)
    except Exception:
        physical = None
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(share, affinity) if share > 0 else affinity
    return {"threads": max(1, threads), "host_logical_cpus": logical, "host_physical_cores": physical,
            "cpus_in_affinity": affinity, "omp_num_threads": share or None}


def _oracle_pass_rate(w, seconds: float, threads: int):
    import oracle

    t0 = time.perf_counter()
    rows = passes = 0
    while True:
        oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"],
                      threads=threads)
        rows += w["B"]
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    return rows / (time.perf_counter() - t0), rows, passes


def cpu_baseline(w, seconds: float, cpus):
    """The oracle on the host: three timed runs of whole passes over the
    benchmark batch, each at least seconds / 3, on cpus["threads"] threads
    (one row per task); the median run is the value."""
    import oracle

    threads = cpus["threads"]
    runs = [_oracle_pass_rate(w, seconds / 3.0, threads) for _ in range(3)]
    rates = sorted(r[0] for r in runs)
    total_rows = sum(r[1] for r in runs)
    # One thread on the first 16 rows, for the single-core figure.
    t1 = time.perf_counter()
    oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"], rows=range(16),
                  threads=1)
    single = 16 / (time.perf_counter() - t1)
    return {"value": rates[1], "unit": "rows/s", "cores": threads, "kind": "oracle",
            "runs_rows_per_s": [r[0] for r in runs], "single_thread_rows_per_s": single, **cpus,
            "sample": f"median of 3 runs, each whole passes over the {w['B']} rows of the benchmark batch for at "
                      f"least {seconds / 3.0:.1f} s ({total_rows} rows in all); float64 stable-sort oracle on "
                      f"{threads} threads (the host's CPU share for one GPU), one row per task; single thread: "
                      f"16 rows"}


def _rotating_buffers(w, dev, nbuf: int = 0):
    """Enough device copies of the batch (> 512 MB in all, or nbuf) that the
    256 MB last-level cache cannot serve a repeat read."""
    import numpy as np
    import torch

    esz = 2 if w["dtype"] == "bf16" else 4
    batch_bytes = w["B"] * w["V"] * esz
    nbuf = nbuf or max(2, -(-(512 * 2**20 + 1) // batch_bytes) + 1)
    if w["dtype"] == "bf16":
        host = torch.from_numpy(w["logits"].view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(w["logits"])
    return [host.to(dev) for _ in range(nbuf)], batch_bytes


def _time_launches(fn, steps: int, warmup: int, stream):
    """Per-launch milliseconds from HIP events recorded on `stream` around each call."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    st = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    en = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        st[i].record(stream)
        fn(warmup + i)
        en[i].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(st, en)], st[0].elapsed_time(en[-1])


def workload_object(n: int, steps: int, warmup: int, dev, stream, cpus, cpu_seconds: float):
    """One workload timed on the library's default path: rows/s, the logits'
    HBM GB/s and fraction of the 8 TB/s peak, per-launch times, and the oracle's
    rows/s over a bounded sample of the same rows."""
    import numpy as np
    import torch

    import nucleus_sampling_amd as ns
    import workloads

    w = workloads.make(n)
    B, V = w["B"], w["V"]
    bufs, batch_bytes = _rotating_buffers(w, dev)
    T, P, K, MP = (torch.from_numpy(w[k]).to(dev) for k in ("temperature", "top_p", "top_k", "min_p"))
    out = ns.SampleResult(torch.empty(B, dtype=torch.int32, device=dev),
                          torch.empty(B, dtype=torch.int32, device=dev), None, None)
    need = ns.workspace_bytes(B, V, bufs[0].dtype)
    ws = ns.workspace_for(dev, stream, need) if need else None

    def step(i):
        ns.sample(bufs[i % len(bufs)], T, P, K, MP, seed=w["seed"], step=i, out=out, workspace=ws, stream=stream)

    ms, span = _time_launches(step, steps, warmup, stream)
    avg = float(np.mean(ms))
    gbps = batch_bytes / (avg * 1e-3) / 1e9
    res = {"workload": f"{w['name']}: B={B}, V={V} {w['dtype']}", "B": B, "V": V, "logit_dtype": w["dtype"],
           "kernel": "tile_kernel" if need else "row_kernel", "steps": steps,
           "avg_launch_ms": avg, "median_launch_ms": float(np.median(ms)),
           "rows_per_s": B / (avg * 1e-3), "rows_per_s_span": B * steps / (span * 1e-3),
           "algorithmic_bytes_per_launch": batch_bytes, "logits_gbps": gbps, "frac_of_hbm_peak": gbps / PEAK_HBM_GBPS}
    if cpu_seconds > 0:
        rate, rows, _ = _oracle_pass_rate(w, cpu_seconds, cpus["threads"])
        res["cpu_oracle_rows_per_s"] = rate
        res["cpu_oracle_sample"] = f"{rows} rows, {cpus['threads']} threads"
    del bufs
    torch.cuda.synchronize()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--buffers", type=int, default=0, help="input copies to rotate (default: > 512 MB total)")
    ap.add_argument("--path", choices=["default", "single", "split", "rows"], default="default",
                    help="force one of the library's paths (for comparisons; the headline uses the default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rejection", action="store_true", help="skip timing the rejection sampler")
    ap.add_argument("--no-spec", action="store_true", help="skip timing speculative verification")
    ap.add_argument("--no-prechain", action="store_true", help="skip timing the pre-chain")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="host seconds for the oracle baseline (three runs of a third each)")
    ap.add_argument("--no-with-probs", action="store_true",
                    help="skip timing the benchmark calls with the probabilities written out")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip timing the other workloads (small, ties, chain, flat)")
    ap.add_argument("--profile-steps", action="store_true", help="only run the timed loop (for rocprofv3)")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="before the timed loop, run a plain elementwise kernel that reads and writes 256 MiB "
                         "(the scale reference for FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of --pmc-calibrate "
                         "--profile-steps into profiles/pmc_<workload>.json and print it")
    args = ap.parse_args()

    if args.pmc_summary:
        import workloads
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], workloads.NAMES[args.workload],
                                     workloads.SHAPES[args.workload], workloads.DTYPES[args.workload]), indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); rows are independent, so a batch "
              "shards across GPUs with no communication; this benchmark measures one GPU.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nucleus_sampling_amd as ns
    import workloads

    ns.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    w = workloads.make(args.workload)
    B, V = w["B"], w["V"]
    bufs, batch_bytes = _rotating_buffers(w, dev, args.buffers)
    nbuf = len(bufs)
    host = bufs[0]
    T = torch.from_numpy(w["temperature"]).to(dev)
    P = torch.from_numpy(w["top_p"]).to(dev)
    K = torch.from_numpy(w["top_k"]).to(dev)
    MP = torch.from_numpy(w["min_p"]).to(dev)
    out = ns.SampleResult(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                          None, None)
    stream = torch.cuda.current_stream(dev)
    flags = {"default": 0, "single": ns.NUCLEUS_FLAG_SINGLE_WORKGROUP, "split": ns.NUCLEUS_FLAG_SPLIT_ROWS,
             "rows": ns.NUCLEUS_FLAG_ROW_RACE}[args.path]
    need = ns.workspace_bytes(B, V, host.dtype, flags)
    ws = ns.workspace_for(dev, stream, need) if need else None
    kernel = {"default": "tile_kernel" if ns.workspace_bytes(B, V, host.dtype) else "row_kernel", "single": "row_kernel",
              "split": "tile_kernel", "rows": "row_kernel+race_kernel"}[args.path]

    def step(i):
        ns.sample(bufs[i % nbuf], T, P, K, MP, seed=w["seed"], step=i, out=out, workspace=ws, stream=stream,
                  single_workgroup=args.path == "single", split_rows=args.path == "split",
                  row_race=args.path == "rows")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.pmc_calibrate:
        cal_src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
        cal_dst = torch.empty_like(cal_src)
        for _ in range(3):
            torch.add(cal_src, 1.0, out=cal_dst)
        torch.cuda.synchronize()
        del cal_src, cal_dst

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    span_ms = starts[0].elapsed_time(ends[-1])
    if args.profile_steps:
        print(json.dumps({"profile_steps": args.steps, "span_ms": span_ms}), flush=True)
        return

    # Pure streaming read of the same buffers: the practical read ceiling.
    sink = torch.zeros(256, dtype=torch.int64, device=dev)
    for i in range(5):
        ns.stream_read(bufs[i % nbuf], sink, stream)
    torch.cuda.synchronize()
    rs = [torch.cuda.Event(enable_timing=True) for _ in range(50)]
    re_ = [torch.cuda.Event(enable_timing=True) for _ in range(50)]
    for i in range(50):
        rs[i].record(stream)
        ns.stream_read(bufs[i % nbuf], sink, stream)
        re_[i].record(stream)
    torch.cuda.synchronize()
    read_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(rs, re_)]))

    # The rejection sampler (nucleus_sample_rejection) on the same buffers:
    # T, top-p and min-p of the workload, top-k off.
    rej = None
    if not args.no_rejection:
        rout = ns.RejectionResult(torch.empty(B, dtype=torch.int32, device=dev),
                                  torch.empty(B, dtype=torch.int32, device=dev))
        for i in range(args.warmup):
            ns.sample_rejection(bufs[i % nbuf], T, P, MP, seed=w["seed"], step=i, out=rout, stream=stream)
        torch.cuda.synchronize()
        js = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        je = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        rounds = []
        for i in range(args.steps):
            js[i].record(stream)
            ns.sample_rejection(bufs[i % nbuf], T, P, MP, seed=w["seed"], step=args.warmup + i, out=rout,
                                stream=stream)
            je[i].record(stream)
            if i < 8:
                rounds.append(rout.rounds.clone())
        torch.cuda.synchronize()
        rj_ms = [a.elapsed_time(e) for a, e in zip(js, je)]
        rr = torch.cat(rounds).float()
        rr = rr[rr > 0]
        rj_avg = float(np.mean(rj_ms))
        rej = {"kernel": "rejection_kernel", "avg_launch_ms": rj_avg, "median_launch_ms": float(np.median(rj_ms)),
               "rows_per_s": B / (rj_avg * 1e-3), "logits_gbps": batch_bytes / (rj_avg * 1e-3) / 1e9,
               "frac_of_hbm_peak": batch_bytes / (rj_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
               "rounds_mean": float(rr.mean()) if rr.numel() else 0.0,
               "rounds_max": int(rr.max()) if rr.numel() else 0,
               "passes_per_row_mean": 2.0 * float(rr.mean()) if rr.numel() else 0.0,
               "note": "top-k off; every row reads its logits 2 x rounds times"}

    # Speculative verification (nucleus_spec_verify) of a synthetic draft
    # against the kept distribution of the first buffer's rows.
    spec = None
    if not args.no_spec:
        q_np, d_np = workloads.make_draft(w, seed=args.workload)
        qd = torch.from_numpy(q_np).to(dev)
        dd = torch.from_numpy(d_np).to(dev)
        pres = ns.sample(bufs[0], T, P, K, MP, seed=w["seed"], step=0, want_probs=True, stream=stream)
        sout = ns.SpecResult(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
        for i in range(args.warmup):
            ns.spec_verify(pres.probs, qd, dd, seed=w["seed"], step=i, out=sout, stream=stream)
        torch.cuda.synchronize()
        ss = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        se = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        acc_rows = 0
        for i in range(args.steps):
            ss[i].record(stream)
            ns.spec_verify(pres.probs, qd, dd, seed=w["seed"], step=args.warmup + i, out=sout, stream=stream)
            se[i].record(stream)
            if i == 0:
                acc_rows = int(sout.accepted.sum())
        torch.cuda.synchronize()
        sp_ms = [a.elapsed_time(e) for a, e in zip(ss, se)]
        sp_avg = float(np.mean(sp_ms))
        # Algorithmic bytes: a rejected row reads its p and q rows (8 B per token).
        sp_bytes = (B - acc_rows) * V * 8 + B * 8
        spec = {"kernel": "spec_kernel", "avg_launch_ms": sp_avg, "median_launch_ms": float(np.median(sp_ms)),
                "rows_per_s": B / (sp_avg * 1e-3), "accepted_rows": acc_rows,
                "algorithmic_bytes_per_launch": sp_bytes,
                "achieved_gbps": sp_bytes / (sp_avg * 1e-3) / 1e9,
                "frac_of_hbm_peak": sp_bytes / (sp_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "note": "draft q = softmax of noisy logits (odd rows truncated to 64 tokens); p from nucleus_sample"}
        del qd, pres

    # The same batch with the pre-chain (history of 256 tokens per row,
    # penalties, a grammar mask forbidding ~20% of the vocabulary).
    prech = None
    if not args.no_prechain:
        pc = workloads.make_prechain(w, hist_len=256, seed=args.workload)
        hist_d = torch.from_numpy(pc["history"]).to(dev)
        rp_d, fp_d, pp_d = (torch.from_numpy(pc[k]).to(dev) for k in ("repetition", "frequency", "presence"))
        am_d = torch.from_numpy(pc["allowed"].view(np.int32)).to(dev)

        def pstep(i):
            ns.sample(bufs[i % nbuf], T, P, K, MP, seed=w["seed"], step=i, out=out, stream=stream, history=hist_d,
                      repetition_penalty=rp_d, frequency_penalty=fp_d, presence_penalty=pp_d, allowed_mask=am_d)

        for i in range(args.warmup):
            pstep(i)
        torch.cuda.synchronize()
        ps_ = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        pe_ = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            ps_[i].record(stream)
            pstep(args.warmup + i)
            pe_[i].record(stream)
        torch.cuda.synchronize()
        pc_ms = [a.elapsed_time(e) for a, e in zip(ps_, pe_)]
        pc_avg = float(np.mean(pc_ms))
        prech = {"kernel": "row_kernel (pre-chain)", "avg_launch_ms": pc_avg, "median_launch_ms": float(np.median(pc_ms)),
                 "rows_per_s": B / (pc_avg * 1e-3), "logits_gbps": batch_bytes / (pc_avg * 1e-3) / 1e9,
                 "frac_of_hbm_peak": batch_bytes / (pc_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                 "note": "history 256 tokens per row, repetition/frequency/presence penalties, mask ~20% forbidden"}

    # The same calls with the renormalised distribution written out
    # (out_probs, B x V fp32): the logits read once plus the probabilities
    # written once.
    with_probs = None
    if args.path == "default" and not args.no_with_probs:
        pout = ns.SampleResult(torch.empty(B, dtype=torch.int32, device=dev),
                               torch.empty(B, dtype=torch.int32, device=dev),
                               torch.empty((B, V), dtype=torch.float32, device=dev), None)

        def prstep(i):
            ns.sample(bufs[i % nbuf], T, P, K, MP, seed=w["seed"], step=i, out=pout, workspace=ws, stream=stream,
                      want_probs=True)

        pr_ms, _ = _time_launches(prstep, args.steps, args.warmup, stream)
        pr_avg = float(np.mean(pr_ms))
        pr_bytes = batch_bytes + B * V * 4
        with_probs = {"kernels": kernel + " (probabilities written in the same launch)", "avg_launch_ms": pr_avg,
                      "median_launch_ms": float(np.median(pr_ms)), "rows_per_s": B / (pr_avg * 1e-3),
                      "algorithmic_bytes_per_launch": pr_bytes,
                      "achieved_gbps": pr_bytes / (pr_avg * 1e-3) / 1e9,
                      "frac_of_hbm_peak": pr_bytes / (pr_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                      "note": "logits read once (4 B per token) + out_probs written once (4 B per token)"}
        del pout

    cpus = host_cpus()
    others = None
    if not args.no_workloads:
        others = {}
        for n in (1, 2, 4, 5):
            if n == args.workload:
                continue
            others[workloads.NAMES[n]] = workload_object(n, args.steps, args.warmup, dev, stream, cpus,
                                                         0.0 if args.no_cpu_baseline else 2.0)

    avg_ms = float(np.mean(per_launch_ms))
    med_ms = float(np.median(per_launch_ms))
    achieved = batch_bytes / (avg_ms * 1e-3) / 1e9
    stream_gbps = batch_bytes / (read_ms * 1e-3) / 1e9
    ms_per_step = span_ms / args.steps
    value = B * args.steps / (span_ms * 1e-3)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w["dtype"] == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w['name']}: B={B}, V={V} {w['dtype']} logits, per-row T/top_p/top_k/min_p",
                   "B": B, "V": V, "logit_dtype": w["dtype"], "input_buffers": nbuf,
                   "input_bytes_per_step": batch_bytes},
        "logits_gbps": achieved,
        "pct_of_hbm_peak": 100.0 * achieved / PEAK_HBM_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic_from_profile(w["name"], batch_bytes),
                     "kernel": kernel, "path": args.path, "avg_launch_ms": avg_ms,
                     "median_launch_ms": med_ms, "p10_launch_ms": float(np.percentile(per_launch_ms, 10)),
                     "p90_launch_ms": float(np.percentile(per_launch_ms, 90)),
                     "algorithmic_bytes_per_launch": batch_bytes},
        "stream_read": {"kernel": "stream_read_kernel", "gbps": stream_gbps, "avg_ms": read_ms,
                        "frac_of_peak": stream_gbps / PEAK_HBM_GBPS, "sampler_vs_stream": achieved / stream_gbps},
        "with_probs": with_probs,
        "workloads": others,
        "rejection": rej,
        "speculative": spec,
        "prechain": prech,
        "wall_s": wall,
        "kernel_hash": kernel_hash(),
    }
    if others:
        for o in others.values():
            o["frac_of_stream_read"] = o["logits_gbps"] / stream_gbps
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, cpus)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
