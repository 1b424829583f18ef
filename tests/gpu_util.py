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
