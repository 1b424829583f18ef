"""nucleus_sample_noalloc (the entry point for callers that cannot allocate
device memory) against nucleus_sample on the same path: two calls in a row
through the C ABI, the second with a smaller batch, each bit-identical to
nucleus_sample's outputs and within the oracle's parity rules."""
import numpy as np
import pytest

import workloads
from gpu_util import device_logits, oracle_and_compare, say

pytestmark = pytest.mark.gpu


def _run(w, noalloc, **kw):
    import torch

    import nucleus_sampling_amd as ns

    lg = device_logits(w["logits"], w["dtype"])
    res = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"], step=3,
                    want_min_kept=True, want_probs=True, noalloc=noalloc, **kw)
    torch.cuda.synchronize()
    return (res.token.cpu().numpy(), res.keep_count.cpu().numpy(), res.min_kept_logit.cpu().numpy(),
            res.probs.cpu().numpy())


@pytest.mark.parametrize("path", [None, "split", "rows"])
def test_noalloc_matches_nucleus_sample(path):
    kw = dict(split_rows=path == "split", row_race=path == "rows")
    # The tie-heavy workload first (64 rows of 32000 tokens: the split-row
    # path's per-chunk slots and lists live in the static scratch), then a
    # smaller batch (the 15-row worked-example workload) reusing the scratch.
    for n in (2, 1):
        w = workloads.make(n)
        say(f"noalloc path={path} workload {n} shape={workloads.SHAPES[n]}")
        got = _run(w, True, **kw)
        want = _run(w, False, **kw)
        for g, e in zip(got, want):
            assert np.array_equal(g, e, equal_nan=True)
        rep, _ = oracle_and_compare(w, got[0], got[1], got[2], step=3, gpu_probs=got[3],
                                    prob_rows=list(range(w["B"])))
        say(f"noalloc path={path} workload {n}: {rep.summary()}")
        assert rep.ok(), rep.failures
