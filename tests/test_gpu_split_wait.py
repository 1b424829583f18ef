"""The split-row path's bounded wait, driven from the host.

The split-row path spreads a row over several workgroups that meet at
per-row barriers in global memory; a wait that cannot end (the row's
workgroups never all running, e.g. when other work holds the device) gives
up after a bounded spin and the row reports token -2, so one failing row
does not hang the batch ("Top-p (Nucleus) Sampling, in depth", "Failure
modes").  A test-only option makes one row's workgroups give up every wait at
once: every kernel must still exit, that row must report -2 with its other
outputs left unwritten, and every other row must match the oracle.  The
next call on the same workspace, without the option, must be whole again.
"""
import numpy as np
import pytest

import workloads
from gpu_util import device_logits, say

pytestmark = pytest.mark.gpu

SENTINEL_COUNT = 777
SENTINEL_PROB = -3.0


def _outputs(B, V, dev):
    import torch

    import nucleus_sampling_amd as ns

    return ns.SampleResult(torch.full((B,), 12345, dtype=torch.int32, device=dev),
                           torch.full((B,), SENTINEL_COUNT, dtype=torch.int32, device=dev),
                           torch.full((B, V), SENTINEL_PROB, dtype=torch.float32, device=dev),
                           torch.full((B,), SENTINEL_PROB, dtype=torch.float32, device=dev), None)


def _compare_rows(w, rows, tok, cnt, mk, probs):
    """Rows `rows` of the batch (their own race counters) against the oracle."""
    import oracle
    from oracle.compare import compare

    rows = np.asarray(rows)
    _, op = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"],
                          rows=rows, want_probs=True, threads=16)
    orows, _ = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"],
                             threads=16)
    return compare(w["logits"][rows], w["temperature"][rows], w["top_p"][rows], w["top_k"][rows],
                   w["min_p"][rows], w["seed"], 0, tok[rows], cnt[rows], mk[rows], orows[rows],
                   gpu_probs=probs[rows], oracle_probs=op, prob_rows=list(range(len(rows))), batch_rows=rows)


@pytest.mark.parametrize("n,give_up", [(2, 5), (2, 0), (4, 255)])
def test_a_row_whose_waits_give_up_reports_minus_two(n, give_up):
    import torch

    import nucleus_sampling_amd as ns

    w = workloads.make(n)
    B, V = w["B"], w["V"]
    lg = device_logits(w["logits"], w["dtype"])
    say(f"workload {n} split rows, row {give_up}'s waits give up at once")
    out = _outputs(B, V, lg.device)
    ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"], want_probs=True,
              want_min_kept=True, split_rows=True, split_give_up_row=give_up, out=out)
    torch.cuda.synchronize()  # every workgroup has exited
    tok, cnt = out.token.cpu().numpy(), out.keep_count.cpu().numpy()
    mk, probs = out.min_kept_logit.cpu().numpy(), out.probs.cpu().numpy()
    assert tok[give_up] == -2
    assert cnt[give_up] == SENTINEL_COUNT and mk[give_up] == SENTINEL_PROB
    assert np.all(probs[give_up] == SENTINEL_PROB)
    others = [b for b in range(B) if b != give_up]
    rep = _compare_rows(w, others, tok, cnt, mk, probs)
    say(f"workload {n}, the other rows: {rep.summary()}")
    assert rep.rows == B - 1
    assert rep.ok(), rep.failures

    say(f"workload {n}: the next call on the same workspace, without the option")
    again = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"], want_probs=True,
                      want_min_kept=True, split_rows=True)
    torch.cuda.synchronize()
    t2, c2, m2, p2 = (again.token.cpu().numpy(), again.keep_count.cpu().numpy(),
                      again.min_kept_logit.cpu().numpy(), again.probs.cpu().numpy())
    assert np.array_equal(t2[others], tok[others]) and np.array_equal(c2[others], cnt[others])
    assert np.array_equal(p2[others].view(np.uint32), probs[others].view(np.uint32))
    rep = _compare_rows(w, [give_up], t2, c2, m2, p2)
    assert rep.ok(), rep.failures


def test_give_up_option_is_checked_on_the_host():
    import torch

    import nucleus_sampling_amd as ns

    lg = torch.zeros((2, 16), device="cuda:0")
    with pytest.raises(ns.NucleusError):
        ns.sample(lg, torch.ones(2), torch.ones(2), split_rows=True, split_give_up_row=-2)
    # Other paths ignore it.
    r = ns.sample(lg, torch.ones(2), torch.full((2,), 0.5), single_workgroup=True, split_give_up_row=0)
    torch.cuda.synchronize()
    assert (r.token.cpu().numpy() >= 0).all()
