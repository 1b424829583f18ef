"""Parity of the fused pre-chain (penalties and grammar mask applied inside
the row kernel's passes) with the oracle: the oracle processes the logits
with oracle_preprocess and runs its sampler on the result; the GPU samples
the raw logits with the pre-chain options.  Rules as for the sampler
(oracle/compare.py)."""
import numpy as np
import pytest

import workloads
from gpu_util import compare_every_row, device_logits, oracle_and_compare, say
from test_gpu_parity import _edge_batch, _random_batch

pytestmark = pytest.mark.gpu


def _gpu(w, pc, lg=None, rows=None, single=False, want_logprobs=False, dev=False):
    """Samples with the pre-chain options; with ``dev`` the result object
    (its tensors on the device), else host arrays with the probabilities of
    ``rows``."""
    import torch

    import nucleus_sampling_amd as ns

    lg = device_logits(w["logits"], w["dtype"]) if lg is None else lg
    res = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"], step=0,
                    want_probs=rows is not None, want_min_kept=True, want_logprobs=want_logprobs,
                    single_workgroup=single, history=pc["history"], repetition_penalty=pc["repetition"],
                    frequency_penalty=pc["frequency"], presence_penalty=pc["presence"],
                    allowed_mask=pc["allowed"].view(np.int32))
    torch.cuda.synchronize()
    if dev:
        return res
    probs = logprobs = None
    if rows is not None:
        idx = torch.as_tensor(list(rows), dtype=torch.long, device=lg.device)
        probs = res.probs.index_select(0, idx).cpu().numpy()
        if want_logprobs:
            logprobs = res.logprobs.index_select(0, idx).cpu().numpy()
    return res.token.cpu().numpy(), res.keep_count.cpu().numpy(), res.min_kept_logit.cpu().numpy(), probs, logprobs


def _processed(w, pc):
    import oracle

    xp = oracle.preprocess(w["logits"], hist=pc["history"], repetition=pc["repetition"], frequency=pc["frequency"],
                           presence=pc["presence"], allowed=pc["allowed"])
    return dict(w, logits=xp, dtype="f32")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_prechain_workload_parity(n):
    """Every row of every workload, its probabilities and log-probabilities
    included, against the oracle's sampler run on the oracle's processed
    logits."""
    say(f"pre-chain, workload {n} ({workloads.NAMES[n]}) shape={workloads.SHAPES[n]}: generating")
    w = workloads.make(n)
    pc = workloads.make_prechain(w, hist_len=1024 if n == 3 else 256, seed=n)
    say(f"pre-chain, workload {n}: sampling on cuda:0")
    lg = device_logits(w["logits"], w["dtype"])
    res = _gpu(w, pc, lg=lg, rows=(), want_logprobs=True, dev=True)
    tok, cnt, mk = res.token.cpu().numpy(), res.keep_count.cpu().numpy(), res.min_kept_logit.cpu().numpy()
    wp = _processed(w, pc)
    say(f"pre-chain, workload {n}: every row against the oracle, 128 rows at a time")
    rep, _ = compare_every_row(wp, tok, cnt, mk, probs_dev=res.probs, logprobs_dev=res.logprobs)
    say(f"pre-chain, workload {n}: {rep.summary()}")
    assert rep.rows == w["B"]
    assert rep.ok(), rep.failures[:10]
    # Never a forbidden token.
    ok = np.nonzero(tok >= 0)[0]
    words = pc["allowed"][ok, tok[ok] // 32]
    assert (((words >> (tok[ok] % 32).astype(np.uint32)) & 1) == 1).all()
    say(f"pre-chain, workload {n}: one workgroup per row on request gives the same bits")
    tok2, cnt2, mk2, _, _ = _gpu(w, pc, lg=lg, single=True)
    assert np.array_equal(tok, tok2) and np.array_equal(cnt, cnt2)
    assert np.array_equal(mk.view(np.uint32), mk2.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 3, 5, 63, 1023, 40001])
def test_prechain_ragged(V, dtype):
    rng = np.random.default_rng(V * 17 + (dtype == "bf16"))
    w = _random_batch(rng, 9, V, dtype)
    pc = workloads.make_prechain(w, hist_len=min(1024, 4 * V + 1), seed=V)
    say(f"pre-chain ragged V={V} {dtype}")
    tok, cnt, mk, probs, _ = _gpu(w, pc, rows=range(9))
    rep, _ = oracle_and_compare(_processed(w, pc), tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(9)))
    assert rep.ok(), rep.failures


def test_prechain_strided_and_edge_rows():
    """Unaligned strided rows (token-by-token loads); the edge rows, where a
    NaN under a forbidden bit is masked away and one under an allowed bit is
    a row error."""
    rng = np.random.default_rng(3)
    B, V, pad = 6, 3001, 3
    w = _random_batch(rng, B, V, "f32")
    pc = workloads.make_prechain(w, hist_len=300, seed=5)
    base = device_logits(np.pad(w["logits"], ((0, 0), (0, pad))), "f32")
    lg = base[:, :V]
    assert lg.stride(0) == V + pad
    tok, cnt, mk, probs, _ = _gpu(w, pc, lg=lg, rows=range(B))
    rep, _ = oracle_and_compare(_processed(w, pc), tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    assert rep.ok(), rep.failures
    L, T, P, K, MP = _edge_batch()
    w = dict(logits=L, dtype="f32", temperature=T, top_p=P, top_k=K, min_p=MP, seed=1, B=len(T), V=L.shape[1])
    pc = workloads.make_prechain(w, hist_len=16, seed=6)
    pc["allowed"][0, 0] &= ~np.uint32(1 << 1)  # row 0's NaN (token 1) is forbidden
    say("pre-chain edge rows")
    tok, cnt, mk, probs, _ = _gpu(w, pc, rows=range(len(T)))
    rep, _ = oracle_and_compare(_processed(w, pc), tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(len(T))))
    say(f"pre-chain edge rows: {rep.summary()}")
    assert rep.ok(), rep.failures
    assert tok[0] >= 0


def _bucket(ids):
    """The kernel's table bucket of each id (multiplicative hash, top 9 bits)."""
    return ((ids.astype(np.uint64) * np.uint64(0x9E3779B1)) & np.uint64(0xFFFFFFFF)) >> np.uint64(23)


def test_prechain_colliding_history():
    """Histories built against the table: one id 1024 times (the largest
    count), 1024 distinct ids from 16 of the 512 buckets (chains of spills
    hundreds of slots long, inserted by 1024 threads at once), colliding ids
    twice each with some of them forbidden, and pads and ids outside [0, V).
    Every token is kept (p = 1), so each token's probability shows its
    processed logit: a lost, doubled or misplaced entry moves it."""
    rng = np.random.default_rng(31)
    B, V, H = 4, 65536, 1024
    L = rng.normal(0.0, 2.0, (B, V)).astype(np.float32)
    ids = np.arange(V)
    near = ids[_bucket(ids) < 16]
    assert len(near) >= H
    hist = np.full((B, H), -1, np.int32)
    hist[0, :] = 777
    hist[1, :] = rng.permutation(near)[:H]
    pair = rng.permutation(near)[:H // 2]
    hist[2, :] = rng.permutation(np.concatenate([pair, pair]))
    hist[3, :600] = rng.integers(0, V, 600)
    hist[3, 600:700] = V + rng.integers(0, 50, 100)
    hist[3, 700:800] = -5
    allow = rng.random((B, V)) >= 0.2
    allow[0, 777] = True                 # the count of 1024 shows
    allow[2, hist[2, : H // 4]] = False  # a quarter of row 2's ids forbidden
    allowed = (allow.reshape(B, V // 32, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(-1)
    allowed = allowed.astype(np.uint32)
    pc = dict(history=hist, repetition=np.full(B, 1.3, np.float32), frequency=np.full(B, 0.05, np.float32),
              presence=np.full(B, 0.2, np.float32), allowed=allowed)
    w = dict(logits=L, dtype="f32", temperature=np.ones(B, np.float32), top_p=np.ones(B, np.float32), top_k=None,
             min_p=None, seed=12, B=B, V=V)
    say("pre-chain colliding histories")
    tok, cnt, mk, probs, _ = _gpu(w, pc, rows=range(B))
    rep, _ = oracle_and_compare(_processed(w, pc), tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    say(f"pre-chain colliding histories: {rep.summary()}")
    assert rep.ok(), rep.failures


def test_prechain_largest_vocabulary():
    """V = 166912, the most the pre-chain stages: the mask fills its LDS
    words to the last one.  Every token's probability against the oracle."""
    rng = np.random.default_rng(41)
    B, V = 4, 166912
    w = _random_batch(rng, B, V, "f32")
    w["top_p"] = np.asarray([1.0, 0.9, 0.5, 1.0], np.float32)
    pc = workloads.make_prechain(w, hist_len=1024, seed=41)
    pc["allowed"][:, -1] = np.uint32(0x0000FFFF)  # the last word's top half forbidden
    say(f"pre-chain V={V}")
    tok, cnt, mk, probs, _ = _gpu(w, pc, rows=range(B))
    rep, _ = oracle_and_compare(_processed(w, pc), tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    say(f"pre-chain V={V}: {rep.summary()}")
    assert rep.ok(), rep.failures
    assert (probs[:, V - 16:] == 0).all()


def test_prechain_rejects_other_paths():
    import torch

    import nucleus_sampling_amd as ns

    lg = torch.zeros((4, 64), device="cuda:0")
    for kw in (dict(split_rows=True), dict(row_race=True)):
        with pytest.raises(ns.NucleusError):
            ns.sample(lg, torch.ones(4), torch.ones(4), allowed_mask=np.zeros((4, 2), np.int32), **kw)
