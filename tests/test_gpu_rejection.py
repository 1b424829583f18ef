"""Parity of the rejection sampler (nucleus_sample_rejection) with the
oracle's rejection sampler, row by row: token and rounds exactly, unless a
round's acceptance test lies within 1e-5 of p or its race within 1e-6 of a
tie (then the token must be admissible under the oracle's masses).  The
tokens are also those of the main sampler on the same inputs (top-k off),
which reaches them through the cut instead.
"""
import numpy as np
import pytest

import workloads
from gpu_util import device_logits, say
from test_gpu_parity import _edge_batch, _random_batch

pytestmark = pytest.mark.gpu


def _rej(w, lg=None, seed=None, step=0, seeds=None):
    import torch

    import nucleus_sampling_amd as ns

    lg = device_logits(w["logits"], w["dtype"]) if lg is None else lg
    res = ns.sample_rejection(lg, w["temperature"], w["top_p"], w["min_p"], seed=w["seed"] if seed is None else seed,
                              step=step, seeds=seeds)
    torch.cuda.synchronize()
    return res.token.cpu().numpy(), res.rounds.cpu().numpy(), lg


def _check(w, tok, rounds, seed=None, step=0, seeds=None, threads=16):
    import oracle
    from oracle.compare import compare_rejection

    s = w["seed"] if seed is None else seed
    orows = oracle.sample_rejection(w["logits"], w["temperature"], w["top_p"], w["min_p"], seed=s, step=step,
                                    seeds=seeds, threads=threads)
    rep = compare_rejection(w["logits"], w["temperature"], w["top_p"], w["min_p"], s, step, tok, rounds, orows,
                            seeds=seeds)
    return rep, orows


def _main_tokens(w, lg, seed=None, step=0, seeds=None):
    import torch

    import nucleus_sampling_amd as ns

    res = ns.sample(lg, w["temperature"], w["top_p"], None, w["min_p"], seed=w["seed"] if seed is None else seed,
                    step=step, seeds=seeds)
    torch.cuda.synchronize()
    return res.token.cpu().numpy()


def _agree_with_main(tok, main, orows):
    """Rows off every boundary draw the main sampler's token."""
    clean = (orows["status"] == 0) & (orows["band"] > 1e-5) & (orows["race_margin"] > 1e-6)
    clean |= orows["status"] == 1
    clean |= orows["greedy"] == 1
    bad = np.nonzero(clean & (tok != main))[0]
    return bad


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_rejection_workload_parity(n):
    say(f"rejection, workload {n} ({workloads.NAMES[n]}) shape={workloads.SHAPES[n]}: generating")
    w = workloads.make(n)
    say(f"rejection, workload {n}: sampling on cuda:0")
    tok, rounds, lg = _rej(w)
    rep, orows = _check(w, tok, rounds)
    say(f"rejection, workload {n}: {rep.summary()}")
    assert rep.ok(), rep.failures[:10]
    say(f"rejection, workload {n}: the main sampler on the same rows (top-k off)")
    bad = _agree_with_main(tok, _main_tokens(w, lg), orows)
    assert len(bad) == 0, bad[:10]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 5, 63, 65, 1023, 4097, 40001])
def test_rejection_ragged_shapes(V, dtype):
    rng = np.random.default_rng(V * 11 + (dtype == "bf16"))
    w = _random_batch(rng, 9, V, dtype)
    say(f"rejection ragged V={V} {dtype}")
    tok, rounds, lg = _rej(w)
    rep, orows = _check(w, tok, rounds)
    assert rep.ok(), rep.failures
    assert len(_agree_with_main(tok, _main_tokens(w, lg), orows)) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rejection_edge_rows(dtype):
    L, T, P, K, MP = _edge_batch()
    if dtype == "bf16":
        L = workloads.f32_to_bf16_bits(L)
    w = dict(logits=L, dtype=dtype, temperature=T, top_p=P, top_k=None, min_p=MP, seed=1)
    say(f"rejection edge rows ({len(T)}) {dtype}")
    tok, rounds, _ = _rej(w)
    rep, _ = _check(w, tok, rounds)
    say(f"rejection edge rows {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rejection_million_token_rows(dtype):
    """Rows of 2^20 + 7 tokens: token and rounds against the oracle, and the
    main sampler's token on rows off every boundary."""
    rng = np.random.default_rng(21 + (dtype == "bf16"))
    w = _random_batch(rng, 3, (1 << 20) + 7, dtype)
    say(f"rejection V={w['V']} {dtype}")
    tok, rounds, lg = _rej(w)
    rep, orows = _check(w, tok, rounds)
    say(f"rejection V={w['V']} {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures
    assert len(_agree_with_main(tok, _main_tokens(w, lg), orows)) == 0


def test_rejection_strided_rows_and_first_race_fallbacks():
    """Unaligned strided rows; rows whose first loaded tokens are all -inf
    (the first round cannot race in the max pass); rows whose max lies far
    above the first tokens' max at a small T (round 1 races again against the
    true max)."""
    rng = np.random.default_rng(5)
    B, V, pad = 8, 70001, 3
    L = rng.normal(0, 1, (B, V)).astype(np.float32)
    L[0, :40000] = -np.inf                    # first buffer all -inf
    L[1, 50000] = 30.0                        # far above the first tokens' max
    L[2, 60000:60003] = 25.0
    L[3, -1] = 9.0
    T = np.asarray([1.0, 0.05, 0.1, 0.2, 0.7, 1.3, 0.0, 2.0], np.float32)
    P = np.asarray([0.9, 0.9, 0.5, 0.95, 0.8, 1.0, 0.9, 0.0], np.float32)
    MP = np.asarray([0.0, 0.0, 0.0, 0.01, 0.0, 0.2, 0.0, 0.0], np.float32)
    w = dict(logits=L, dtype="f32", temperature=T, top_p=P, top_k=None, min_p=MP, seed=77)
    base = device_logits(np.pad(L, ((0, 0), (0, pad))), "f32")
    lg = base[:, :V]
    assert lg.stride(0) == V + pad
    say("rejection strided rows / first-race fallbacks")
    tok, rounds, _ = _rej(w, lg=lg)
    rep, orows = _check(w, tok, rounds)
    say(f"rejection strided: {rep.summary()}")
    assert rep.ok(), rep.failures
    assert tok[1] == 50000 and tok[2] in (60000, 60001, 60002)
    assert len(_agree_with_main(tok, _main_tokens(w, lg), orows)) == 0


def test_rejection_seeds_and_steps():
    """Per-row keys and the step: rows draw with their own key, and a new step
    changes the draws."""
    rng = np.random.default_rng(8)
    B, V = 32, 5000
    L = rng.normal(0, 1.5, (B, V)).astype(np.float32)
    w = dict(logits=L, dtype="f32", temperature=np.full(B, 1.2, np.float32),
             top_p=np.full(B, 0.95, np.float32), top_k=None, min_p=None, seed=3)
    seeds = rng.integers(0, 2**63, B, dtype=np.uint64)
    say("rejection per-row seeds")
    tok, rounds, lg = _rej(w, seeds=seeds, step=9)
    rep, orows = _check(w, tok, rounds, step=9, seeds=seeds)
    assert rep.ok(), rep.failures
    assert len(_agree_with_main(tok, _main_tokens(w, lg, step=9, seeds=seeds), orows)) == 0
    tok2, _, _ = _rej(w, seeds=seeds, step=10)
    assert (tok2 != tok).sum() > B // 2


def test_rejection_empty_batch():
    import torch

    import nucleus_sampling_amd as ns

    lg = torch.zeros((0, 11), device="cuda:0")
    res = ns.sample_rejection(lg, torch.zeros(0), torch.zeros(0))
    torch.cuda.synchronize()
    assert res.token.numel() == 0


def test_rejection_long_chains():
    """Zipf rows with p of 0, 1e-4 and 0.01 need many rounds: the first
    proposals come from round 1's list of high scores, the rest from race
    passes over the tokens above the pivot.  Token and rounds must still match
    the oracle's sequential rounds."""
    w = workloads.make(3, rows=range(64))
    B = w["B"]
    w["top_p"] = np.asarray([[0.0, 1e-4, 0.01, 0.05][b % 4] for b in range(B)], np.float32)
    say("rejection long chains")
    tok, rounds, lg = _rej(w)
    rep, orows = _check(w, tok, rounds)
    say(f"rejection long chains: {rep.summary()}")
    assert rep.ok(), rep.failures[:10]
    assert rounds.max() > 4  # past the list's four proposals
    assert len(_agree_with_main(tok, _main_tokens(w, lg), orows)) == 0
