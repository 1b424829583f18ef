"""Where the one-workgroup-per-row kernel spends its time, row by row.

    python -m nucleus_sampling_amd.phase_stamps [--workload 3] [--calls 5] [--probs]

Loads libnucleus_stamps.so (built by `python -m nucleus_sampling_amd.build
--stamps`: the product library with phase clocks compiled in), samples a
workload from workloads.py on its default path, and reads the clocks thread 0
of every row's workgroup wrote at the phase boundaries of the last call
(include/nucleus.h, nucleus_phase_stamps).  The calls rotate over copies of
the batch (> 512 MB in all), so the measured call reads from HBM.  Prints,
per phase, the median over all rows, over the rows that keep more than 8192
tokens and the maximum, in microseconds, and the phases of the row that ends
last.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

PHASES = [("pass 1 (max + fused histogram)", 0, 1), ("bins ready (fold or pass 2)", 1, 2), ("decide", 2, 3),
          ("classify", None, 4), ("pass 3 (race + candidates)", 4, 5), ("resolver + outputs", 5, 6),
          ("probabilities", 6, 7)]
TICK_US = 0.01  # the 100 MHz constant-rate clock


def row_phases(st: np.ndarray):
    """[B, 8] clocks -> dict phase -> [B] microseconds (NaN where a row skips the phase)."""
    s = st.astype(np.float64)
    s[st == 0] = np.nan
    out = {}
    for name, a, b in PHASES:
        if a is None:  # classify follows decide, or pass 1 for rows without bins
            prev = np.where(np.isnan(s[:, 3]), s[:, 1], s[:, 3])
            out[name] = (s[:, b] - prev) * TICK_US
        else:
            out[name] = (s[:, b] - s[:, a]) * TICK_US
    out["the row"] = (s[:, 7] - s[:, 0]) * TICK_US
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--calls", type=int, default=5)
    ap.add_argument("--probs", action="store_true", help="also write the probabilities (pass 4)")
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    import torch

    import nucleus_sampling_amd as ns
    import workloads
    from nucleus_sampling_amd.build import LIB_STAMPS

    if not os.path.exists(LIB_STAMPS):
        raise SystemExit(f"{LIB_STAMPS} is missing: build it with `python -m nucleus_sampling_amd.build --stamps`")
    ns.LIB_PATH = LIB_STAMPS
    L = ns.lib()
    dev = torch.device("cuda:0")
    w = workloads.make(args.workload)
    B, V = w["B"], w["V"]
    host = (torch.from_numpy(w["logits"].view(np.int16)).view(torch.bfloat16) if w["dtype"] == "bf16"
            else torch.from_numpy(w["logits"]))
    nbuf = max(2, -(-(512 * 2**20 + 1) // (host.numel() * host.element_size())) + 1)
    bufs = [host.to(dev) for _ in range(nbuf)]
    stamps = torch.zeros((B, 16), dtype=torch.int64, device=dev)
    rc = L.nucleus_phase_stamps(stamps.data_ptr(), B)
    if rc != 0:
        raise SystemExit(f"nucleus_phase_stamps: {ns.strerror(rc)}")
    T, P, K, MP = (torch.from_numpy(w[k]).to(dev) for k in ("temperature", "top_p", "top_k", "min_p"))
    for i in range(args.calls):
        if i == args.calls - 1:
            torch.cuda.synchronize()
            stamps.zero_()
        r = ns.sample(bufs[i % nbuf], T, P, K, MP, seed=w["seed"], step=i, single_workgroup=True,
                      want_probs=args.probs)
    torch.cuda.synchronize()
    L.nucleus_phase_stamps(None, 0)
    full = stamps.cpu().numpy().view(np.uint64)
    st = full[:, :8]
    kept = r.keep_count.cpu().numpy()
    ph = row_phases(st)
    dense = kept > 8192
    span = (np.nanmax(st[:, 7].astype(np.float64)) - np.nanmin(st[:, 0].astype(np.float64))) * TICK_US
    last = int(np.nanargmax(st[:, 7].astype(np.float64)))
    rows = []
    for name in [p[0] for p in PHASES] + ["the row"]:
        v = ph[name]
        rows.append({"phase": name, "median_us": float(np.nanmedian(v)) if np.isfinite(v).any() else None,
                     "median_dense_us": float(np.nanmedian(v[dense])) if np.isfinite(v[dense]).any() else None,
                     "max_us": float(np.nanmax(v)) if np.isfinite(v).any() else None,
                     "last_row_us": float(v[last]) if np.isfinite(v[last]) else None})
    res_us = ph["resolver + outputs"]
    slow = [int(i) for i in np.argsort(-np.nan_to_num(res_us, nan=-1.0))[:5]]
    res = {"workload": f"{w['name']}: B={B}, V={V} {w['dtype']}", "calls": args.calls, "probs": args.probs,
           "launch_span_us": span, "rows_keeping_more_than_8192": int(dense.sum()),
           "last_row": {"row": last, "keep_count": int(kept[last])}, "phases": rows,
           "slowest_resolvers": [{"row": i, "us": float(res_us[i]), "mode": int(full[i, 8]),
                                  "candidates": int(full[i, 9]), "marked_groups": int(full[i, 10]),
                                  "keep_count": int(kept[i]), "T": float(w["temperature"][i]),
                                  "p": float(w["top_p"][i])} for i in slow]}
    if args.json:
        print(json.dumps(res))
        return
    print(f"{res['workload']}: launch span {span:.1f} us (first start to last end), "
          f"{int(dense.sum())} rows keep > 8192 tokens; row {last} (keeps {int(kept[last])}) ends last")
    print(f"{'phase':34s} {'median':>8s} {'dense':>8s} {'max':>8s} {'last row':>9s}")

    def f(x):
        return f"{x:8.1f}" if x is not None else "       -"

    for r_ in rows:
        print(f"{r_['phase']:34s} {f(r_['median_us'])} {f(r_['median_dense_us'])} {f(r_['max_us'])} "
              f"{f(r_['last_row_us'])} ")
    print("slowest resolvers: " + "; ".join(
        f"row {s['row']} {s['us']:.1f} us (mode {s['mode']}, {s['candidates']} candidates in {s['marked_groups']} "
        f"marked groups, keeps {s['keep_count']}, T {s['T']:.2f}, p {s['p']:.4f})" for s in res["slowest_resolvers"]))


if __name__ == "__main__":
    main()
