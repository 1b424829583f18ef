"""Helpers for the GPU tests: move seeded inputs to the device, call the
library through its binding, and bring the outputs back."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def device_logits(logits_np, dtype):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(logits_np).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32))
    return t.to("cuda:0")


def run_gpu(w, step=0, want_probs=False, logits_dev=None, seed=None):
    """Sample workload dict ``w`` on cuda:0; returns numpy (token, count, min_kept, probs)."""
    import torch

    import nucleus_sampling_amd as ns

    lg = logits_dev if logits_dev is not None else device_logits(w["logits"], w["dtype"])
    res = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"],
                    seed=w["seed"] if seed is None else seed, step=step, want_probs=want_probs,
                    want_min_kept=True)
    torch.cuda.synchronize()
    probs = res.probs.cpu().numpy() if res.probs is not None else None
    return res.token.cpu().numpy(), res.keep_count.cpu().numpy(), res.min_kept_logit.cpu().numpy(), probs


def oracle_and_compare(w, tok, cnt, mk, step=0, gpu_probs=None, prob_rows=None, threads=16, seed=None,
                       seeds=None, gpu_logprobs=None):
    import oracle
    from oracle.compare import compare

    s = w["seed"] if seed is None else seed
    rows, oprobs = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=s,
                                 step=step, threads=threads, seeds=seeds)
    op = ol = None
    if prob_rows is not None:
        _, op, ol = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=s,
                                  step=step, rows=prob_rows, want_probs=True, threads=threads, seeds=seeds,
                                  want_logprobs=True)
    rep = compare(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], s, step, tok, cnt, mk,
                  rows, gpu_probs=gpu_probs, oracle_probs=op, prob_rows=prob_rows, seeds=seeds,
                  gpu_logprobs=gpu_logprobs, oracle_logprobs=ol)
    return rep, rows


def _merge(total, rep, r0):
    for f in ("rows", "exact", "errors_ok", "greedy", "exempt_mass", "exempt_mass_exact", "exempt_race",
              "exempt_minp", "near_1e6", "near_1e7"):
        setattr(total, f, getattr(total, f) + getattr(rep, f))
    total.max_prob_ratio = max(total.max_prob_ratio, rep.max_prob_ratio)
    total.max_logprob_ratio = max(total.max_logprob_ratio, rep.max_logprob_ratio)
    total.failures.extend((b + r0, why) for b, why in rep.failures)


def compare_every_row(w, tok, cnt, mk, probs_dev=None, logprobs_dev=None, step=0, seed=None, seeds=None, chunk=128,
                      threads=16):
    """Every row of a batch against the oracle, with its probabilities and
    log-probabilities when the device tensors are given, a chunk of rows at a
    time: the oracle's float64 arrays for a whole 1024 x 152064 batch alone
    would take 2.5 GB of host memory.  Each chunk keeps its rows' own indices
    (the race counter) and keys.  Returns (Report over the batch, the
    oracle's rows)."""
    import oracle
    from oracle import ROW_DTYPE
    from oracle.compare import Report, compare

    B = w["B"]
    s = w["seed"] if seed is None else seed
    T, P = np.asarray(w["temperature"], np.float32), np.asarray(w["top_p"], np.float32)
    K = np.zeros(B, np.int32) if w.get("top_k") is None else np.asarray(w["top_k"], np.int32)
    MP = np.zeros(B, np.float32) if w.get("min_p") is None else np.asarray(w["min_p"], np.float32)
    total, orows = Report(), np.zeros(B, ROW_DTYPE)
    want_p, want_l = probs_dev is not None, logprobs_dev is not None
    for r0 in range(0, B, chunk):
        r1 = min(B, r0 + chunk)
        sl = slice(r0, r1)
        res = oracle.sample(w["logits"], T, P, K, MP, seed=s, step=step, rows=range(r0, r1), want_probs=want_p,
                            threads=threads, seeds=seeds, want_logprobs=want_l)
        o, op = res[0], res[1]
        ol = res[2] if want_l else None
        orows[sl] = o[sl]
        gp = probs_dev[r0:r1].cpu().numpy() if want_p else None
        gl = logprobs_dev[r0:r1].cpu().numpy() if want_l else None
        rep = compare(w["logits"][sl], T[sl], P[sl], K[sl], MP[sl], s, step, tok[sl], cnt[sl],
                      None if mk is None else mk[sl], o[sl], gpu_probs=gp, oracle_probs=op,
                      prob_rows=list(range(r1 - r0)) if (want_p or want_l) else None,
                      batch_rows=np.arange(r0, r1), seeds=None if seeds is None else seeds[sl], gpu_logprobs=gl,
                      oracle_logprobs=ol)
        _merge(total, rep, r0)
    return total, orows
