"""Parity of speculative verification (nucleus_spec_verify) with the oracle:
the GPU takes nucleus_sample's kept distribution p and a draft distribution
q, the oracle derives p from the logits itself; acceptance and the residual
draw must agree row by row under the rules of oracle/compare.py
(compare_spec)."""
import numpy as np
import pytest

import workloads
from gpu_util import device_logits, say
from test_gpu_parity import _edge_batch, _random_batch

pytestmark = pytest.mark.gpu


def _run(w, q, d, seed=None, step=0, seeds=None, lg=None):
    import torch

    import nucleus_sampling_amd as ns

    lg = device_logits(w["logits"], w["dtype"]) if lg is None else lg
    s = w["seed"] if seed is None else seed
    res = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=s, step=step, want_probs=True,
                    seeds=seeds)
    qd = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(lg.device)
    dd = torch.from_numpy(np.ascontiguousarray(d, np.int32)).to(lg.device)
    sp = ns.spec_verify(res.probs, qd, dd, seed=s, step=step, seeds=seeds)
    torch.cuda.synchronize()
    tok = sp.token.cpu().numpy()
    idx = torch.from_numpy(np.clip(tok, 0, q.shape[1] - 1).astype(np.int64)).to(lg.device)
    p_at = res.probs.gather(1, idx[:, None])[:, 0].cpu().numpy()
    return tok, sp.accepted.cpu().numpy(), res.keep_count.cpu().numpy(), p_at


def _check(w, q, d, tok, acc, cnt, p_at, seed=None, step=0, seeds=None):
    import oracle
    from oracle.compare import SPEC_REL_TOL, compare_spec

    s = w["seed"] if seed is None else seed
    orows = oracle.spec_verify(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], q, d, seed=s,
                               step=step, seeds=seeds, rel_tol=SPEC_REL_TOL, threads=16)
    otarget, _ = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=s, step=step,
                               threads=16, seeds=seeds)
    return compare_spec(q, d, tok, acc, cnt, p_at, orows, otarget, w["top_p"])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_spec_workload_parity(n):
    say(f"speculative, workload {n} ({workloads.NAMES[n]}) shape={workloads.SHAPES[n]}: generating")
    w = workloads.make(n)
    q, d = workloads.make_draft(w, seed=n)
    say(f"speculative, workload {n}: target probabilities and verification on cuda:0")
    tok, acc, cnt, p_at = _run(w, q, d)
    rep = _check(w, q, d, tok, acc, cnt, p_at)
    say(f"speculative, workload {n}: {rep.summary()}")
    assert rep.ok(), rep.failures[:10]
    assert rep.exact > 0.8 * rep.rows


@pytest.mark.parametrize("V", [1, 3, 5, 63, 1023, 4097, 40001])
def test_spec_ragged_shapes(V):
    rng = np.random.default_rng(V * 13)
    w = _random_batch(rng, 9, V, "f32")
    q, d = workloads.make_draft(w, keep_top=max(1, V // 3), seed=V)
    say(f"speculative ragged V={V}")
    tok, acc, cnt, p_at = _run(w, q, d)
    rep = _check(w, q, d, tok, acc, cnt, p_at)
    assert rep.ok(), rep.failures


def test_spec_million_token_rows():
    """Rows of 2^20 + 7 tokens: 129 chunks of 8192 per row, the last one
    ragged."""
    rng = np.random.default_rng(22)
    w = _random_batch(rng, 3, (1 << 20) + 7, "f32")
    q, d = workloads.make_draft(w, keep_top=4096, seed=22)
    say(f"speculative V={w['V']}")
    tok, acc, cnt, p_at = _run(w, q, d)
    rep = _check(w, q, d, tok, acc, cnt, p_at)
    say(f"speculative V={w['V']}: {rep.summary()}")
    assert rep.ok(), rep.failures


def test_spec_edge_rows_and_bad_drafts():
    """Target row errors (p all zero), greedy targets, ties, and draft tokens
    outside [0, V)."""
    L, T, P, K, MP = _edge_batch()
    w = dict(logits=L, dtype="f32", temperature=T, top_p=P, top_k=K, min_p=MP, seed=1)
    q, d = workloads.make_draft(w, keep_top=5, seed=9)
    d[3] = -1
    d[5] = L.shape[1]
    say(f"speculative edge rows ({len(T)})")
    tok, acc, cnt, p_at = _run(w, q, d)
    rep = _check(w, q, d, tok, acc, cnt, p_at)
    say(f"speculative edge rows: {rep.summary()}")
    assert rep.ok(), rep.failures
    assert tok[3] == -1 and tok[5] == -1


def test_spec_row_seeds_and_draft_equal_target():
    """Per-row keys; a draft equal to the target's own p is always accepted."""
    import torch

    import nucleus_sampling_amd as ns

    rng = np.random.default_rng(21)
    B, V = 24, 3000
    L = rng.normal(0, 2, (B, V)).astype(np.float32)
    w = dict(logits=L, dtype="f32", temperature=np.full(B, 0.9, np.float32), top_p=np.full(B, 0.9, np.float32),
             top_k=None, min_p=None, seed=4)
    seeds = rng.integers(0, 2**63, B, dtype=np.uint64)
    q, d = workloads.make_draft(w, seed=2)
    say("speculative per-row seeds")
    tok, acc, cnt, p_at = _run(w, q, d, step=3, seeds=seeds)
    rep = _check(w, q, d, tok, acc, cnt, p_at, step=3, seeds=seeds)
    assert rep.ok(), rep.failures
    lg = device_logits(L, "f32")
    res = ns.sample(lg, w["temperature"], w["top_p"], None, None, seed=4, step=3, want_probs=True)
    dd = res.token.clone()
    sp = ns.spec_verify(res.probs, res.probs.clone(), dd, seed=4, step=3)
    torch.cuda.synchronize()
    assert (sp.accepted.cpu().numpy() == 1).all()
    assert np.array_equal(sp.token.cpu().numpy(), dd.cpu().numpy())
