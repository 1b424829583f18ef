"""Parity of the HIP sampler with the float64 oracle, element by element.

Every test calls the library through its C ABI (via the ctypes binding) on
cuda:0 with seeded inputs from workloads.py, and compares with the oracle
under the rules of oracle/compare.py: exact keep sets, keep counts and
tokens; probabilities within 1e-6 + 1e-5 p; rows within 1e-5 of a mass
boundary or 1e-6 of a race tie judged by the admissible-set rule.
"""
import numpy as np
import pytest

import workloads
from gpu_util import compare_every_row, device_logits, oracle_and_compare, say

pytestmark = pytest.mark.gpu


# The library's paths: None = its own choice for the batch; "single" = one
# workgroup per row for everything; "split" = rows split over
# register-resident workgroups; "rows" = a workgroup per row for the
# histogram passes with the race spread over chunks.
PATHS = [None, "single", "split", "rows"]


def _gpu(w, step=0, want_probs=False, prob_rows=None, seed=None, lg=None, path=None, seeds=None,
         want_logprobs=False):
    import torch

    import nucleus_sampling_amd as ns

    lg = device_logits(w["logits"], w["dtype"]) if lg is None else lg
    res = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"],
                    seed=w["seed"] if seed is None else seed, step=step, want_probs=want_probs, want_min_kept=True,
                    single_workgroup=path == "single", split_rows=path == "split", row_race=path == "rows",
                    seeds=seeds, want_logprobs=want_logprobs)
    torch.cuda.synchronize()
    probs = logprobs = None
    if want_probs or want_logprobs:
        idx = torch.as_tensor(list(prob_rows), dtype=torch.long, device=lg.device)
        if want_probs:
            probs = res.probs.index_select(0, idx).cpu().numpy()
        if want_logprobs:
            logprobs = res.logprobs.index_select(0, idx).cpu().numpy()
    out = (res.token.cpu().numpy(), res.keep_count.cpu().numpy(), res.min_kept_logit.cpu().numpy(), probs)
    return out + (logprobs,) if want_logprobs else out


def _gpu_dev(w, step=0, want_probs=False, seed=None, lg=None, path=None, seeds=None, want_logprobs=False):
    """One call; the result's tensors stay on the device."""
    import torch

    import nucleus_sampling_amd as ns

    lg = device_logits(w["logits"], w["dtype"]) if lg is None else lg
    res = ns.sample(lg, w["temperature"], w["top_p"], w["top_k"], w["min_p"],
                    seed=w["seed"] if seed is None else seed, step=step, want_probs=want_probs, want_min_kept=True,
                    single_workgroup=path == "single", split_rows=path == "split", row_race=path == "rows",
                    seeds=seeds, want_logprobs=want_logprobs)
    torch.cuda.synchronize()
    return res


def _host(res):
    return res.token.cpu().numpy(), res.keep_count.cpu().numpy(), res.min_kept_logit.cpu().numpy()


def _same_bits(a, b):
    """Two device tensors hold the same bits (NaN included)."""
    import torch

    return a.shape == b.shape and bool(torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32)))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_parity(n):
    """Every row of every workload against the oracle: keep set, token and
    the renormalised probabilities of all V tokens."""
    say(f"workload {n} ({workloads.NAMES[n]}) shape={workloads.SHAPES[n]} {workloads.DTYPES[n]}: generating")
    w = workloads.make(n)
    lg = device_logits(w["logits"], w["dtype"])
    say(f"workload {n}: sampling on cuda:0 (no probs: the benchmark's launch)")
    tok, cnt, mk = _host(_gpu_dev(w, lg=lg))
    say(f"workload {n}: sampling with probabilities")
    res = _gpu_dev(w, lg=lg, want_probs=True)
    tok2, cnt2, mk2 = _host(res)
    assert np.array_equal(tok, tok2) and np.array_equal(cnt, cnt2)
    assert np.array_equal(mk.view(np.uint32), mk2.view(np.uint32))
    say(f"workload {n}: every row and its probabilities against the oracle, 128 rows at a time")
    rep, _ = compare_every_row(w, tok2, cnt2, mk2, probs_dev=res.probs)
    say(f"workload {n}: {rep.summary()}")
    assert rep.rows == w["B"]
    assert rep.ok(), rep.failures


def _random_batch(rng, B, V, dtype, extras=True):
    kind = rng.integers(0, 3, B)
    L = np.empty((B, V), np.float32)
    for b in range(B):
        if kind[b] == 0:
            L[b] = rng.normal(0, 2, V)
        elif kind[b] == 1:
            L[b] = rng.integers(-2, 3, V)
        else:
            L[b] = -1.1 * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)
        if rng.random() < 0.3:
            L[b, rng.random(V) < 0.2] = -np.inf
            L[b, rng.integers(0, V)] = 0.5
    T = rng.choice([0.0, 0.3, 0.7, 1.0, 1.5, 3.0], B).astype(np.float32)
    P = np.where(rng.random(B) < 0.15, 1.0, rng.uniform(0.05, 0.999, B)).astype(np.float32)
    K = (np.where(rng.random(B) < 0.4, rng.integers(1, V + 3, B), 0) if extras else np.zeros(B)).astype(np.int32)
    MP = (np.where(rng.random(B) < 0.3, rng.uniform(0, 0.5, B), 0.0) if extras else np.zeros(B)).astype(np.float32)
    logits = workloads.f32_to_bf16_bits(L) if dtype == "bf16" else L
    return dict(logits=logits, dtype=dtype, temperature=T, top_p=P, top_k=K, min_p=MP, seed=4242, B=B, V=V)


@pytest.mark.parametrize("path", [None, "rows", "single"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_million_token_rows(dtype, path):
    """Rows of 2^20 + 7 tokens, far past any workload's vocabulary (513
    chunked-race items of 2048 tokens per row, the last one ragged; the
    default path takes one workgroup per row, rows this long being past the
    split-row limit).  Every token's probability against the oracle."""
    rng = np.random.default_rng(20 + (dtype == "bf16"))
    B, V = 3, (1 << 20) + 7
    w = _random_batch(rng, B, V, dtype)
    say(f"V={V} {dtype} B={B} path={path}")
    tok, cnt, mk, probs = _gpu(w, want_probs=True, prob_rows=range(B), path=path)
    rep, _ = oracle_and_compare(w, tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    say(f"V={V} {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_rows_at_their_limit(dtype):
    """The split-row path at its longest rows (64 workgroups of 8192 tokens,
    V = 524288) against the oracle; one token more and the split flag is
    refused."""
    rng = np.random.default_rng(64 + (dtype == "bf16"))
    B, V = 3, 64 * 8192
    w = _random_batch(rng, B, V, dtype)
    say(f"split rows V={V} {dtype}")
    tok, cnt, mk, probs = _gpu(w, want_probs=True, prob_rows=range(B), path="split")
    rep, _ = oracle_and_compare(w, tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    say(f"split rows V={V} {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures
    import nucleus_sampling_amd as ns

    w1 = _random_batch(rng, 2, V + 1, dtype)
    with pytest.raises(ns.NucleusError):
        _gpu(w1, path="split")


@pytest.mark.parametrize("path", [None, "rows", "single", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 3, 5, 63, 64, 65, 1023, 4097, 9999, 40001])
def test_small_and_ragged_shapes(V, dtype, path):
    rng = np.random.default_rng(V * 7 + (dtype == "bf16"))
    B = 9
    w = _random_batch(rng, B, V, dtype)
    say(f"ragged V={V} {dtype} B={B} path={path}")
    tok, cnt, mk, probs = _gpu(w, want_probs=True, prob_rows=range(B), path=path)
    rep, _ = oracle_and_compare(w, tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    say(f"ragged V={V} {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("path", [None, "rows", "single", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_unaligned_rows(dtype, path):
    """Rows whose starts are not 16-byte aligned take the scalar-load path."""
    import torch

    rng = np.random.default_rng(17)
    B, V, pad = 6, 3001, 3
    w = _random_batch(rng, B, V, dtype)
    say(f"strided rows V={V} stride={V + pad} {dtype} path={path}")
    base = device_logits(np.pad(w["logits"], ((0, 0), (0, pad))), dtype)
    lg = base[:, :V]
    assert lg.stride(0) == V + pad
    tok, cnt, mk, probs = _gpu(w, want_probs=True, prob_rows=range(B), lg=lg, path=path)
    rep, _ = oracle_and_compare(w, tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(B)))
    assert rep.ok(), rep.failures
    torch.cuda.synchronize()


def _edge_batch():
    V = 37
    inf, nan = np.inf, np.nan
    rows, T, P, K, MP = [], [], [], [], []

    def add(row, t=1.0, p=0.9, k=0, mp=0.0):
        r = np.full(V, -inf, np.float32)
        r[: len(row)] = row
        rows.append(r); T.append(t); P.append(p); K.append(k); MP.append(mp)

    add([1.0, nan, 2.0])                      # NaN logit
    add([1.0, inf, 2.0])                      # +inf logit
    add([])                                   # no finite logit
    add([1.0, 2.0], t=nan)                    # NaN parameters
    add([1.0, 2.0], p=nan)
    add([1.0, 2.0], mp=nan)
    add([1.0, nan], t=0.0)                    # greedy rows still fail on NaN
    add([3.0, 5.0, 5.0, 1.0], t=0.0)          # greedy, lowest index on ties
    add([3.0, 5.0, 5.0, 1.0], t=-2.0)
    add([0.5, 0.25, 3.0], p=1.0)              # p >= 1 keeps every finite token
    add([0.5, 0.25, 3.0], p=7.0)
    add([1.0, 2.0, 2.0, 0.0], p=0.0)          # p <= 0 keeps the top level
    add([1.0, 2.0, 2.0, 0.0], p=-1.0)
    add([1.0, 2.0, 2.0, 0.0], p=1e-8)
    add([4.0, 1.0, 4.0, 3.9], p=1.0, k=1)     # top-k = 1 keeps tied maxima
    add([4.0, 1.0, 3.0, 2.0], p=1.0, k=2)
    add([4.0, 1.0, 3.0, 2.0], p=1.0, k=100)
    add([4.0, 1.0, 3.0, 2.0], p=1.0, k=-4)
    add(list(np.log([0.5, 0.25, 0.125, 0.0625, 0.0625])), p=1.0, mp=0.3)
    add(list(np.log([0.5, 0.25, 0.125, 0.0625, 0.0625])), p=1.0, mp=5.0)
    add(list(np.log([0.5, 0.25, 0.125, 0.0625, 0.0625])), p=1.0, mp=1e-30)
    add([0.0, -0.0, -1.0], p=0.3)             # -0.0 and +0.0 are one level
    add([2.0, 1.0, 0.0], t=np.inf, p=0.5)     # T = +inf: uniform over finite tokens
    add([2.0, 1.0, 0.0], t=np.inf, p=1.0, mp=1.0)
    add([2.0, 1.9999999, 0.0], t=1e-30)       # tiny T
    add([2.0, 1.0, 0.0], t=1e-44)             # subnormal T
    add([3e38, -3e38, 0.0], p=0.999)          # x - max overflows fp32
    add([3e38, 3e38, -3e38], p=0.5)
    add([1e-40, 0.0, -1e-40], t=1e-38)        # subnormal logits
    add([7.0])                                # a single finite token
    add(list(np.linspace(1.0, 0.0, 37)), p=0.9999999)
    add([1.0] * 37, p=0.3)                    # one level
    add([1.0] * 37, p=0.3, k=5)
    return np.stack(rows), np.asarray(T, np.float32), np.asarray(P, np.float32), np.asarray(K, np.int32), \
        np.asarray(MP, np.float32)


@pytest.mark.parametrize("path", [None, "rows", "single", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_rows(dtype, path):
    L, T, P, K, MP = _edge_batch()
    if dtype == "bf16":
        L = workloads.f32_to_bf16_bits(L)
    w = dict(logits=L, dtype=dtype, temperature=T, top_p=P, top_k=K, min_p=MP, seed=1, B=len(T), V=L.shape[1])
    say(f"edge rows ({len(T)}) {dtype} path={path}")
    tok, cnt, mk, probs = _gpu(w, want_probs=True, prob_rows=range(len(T)), path=path)
    rep, _ = oracle_and_compare(w, tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(len(T))))
    say(f"edge rows {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures


@pytest.mark.parametrize("path", PATHS)
def test_single_column(path):
    rng = np.random.default_rng(2)
    w = _random_batch(rng, 5, 1, "f32")
    tok, cnt, mk, probs = _gpu(w, want_probs=True, prob_rows=range(5), path=path)
    rep, _ = oracle_and_compare(w, tok, cnt, mk, gpu_probs=probs, prob_rows=list(range(5)))
    assert rep.ok(), rep.failures


def test_empty_batch():
    import torch

    import nucleus_sampling_amd as ns

    say("empty batch")
    lg = torch.zeros((0, 11), device="cuda:0")
    res = ns.sample(lg, torch.zeros(0), torch.zeros(0))
    torch.cuda.synchronize()
    assert res.token.numel() == 0


def test_determinism_step_and_row_independence():
    rng = np.random.default_rng(99)
    w = _random_batch(rng, 32, 5000, "f32", extras=False)
    w["temperature"][:] = 1.0
    w["top_p"][:] = 0.97
    say("determinism: repeated calls")
    a = _gpu(w)
    b = _gpu(w)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3]))
    say("determinism: a new step changes the draws")
    c = _gpu(w, step=1)
    assert (a[0] != c[0]).sum() >= 8
    rep, _ = oracle_and_compare(w, *c[:3], step=1)
    assert rep.ok(), rep.failures
    say("row independence: other rows changed")
    w2 = dict(w)
    w2["logits"] = w["logits"].copy()
    w2["logits"][1::2] = rng.normal(0, 1, w2["logits"][1::2].shape).astype(np.float32)
    d = _gpu(w2)
    assert np.array_equal(a[0][0::2], d[0][0::2]) and np.array_equal(a[1][0::2], d[1][0::2])


def test_draws_match_oracle_on_worked_example():
    """20,000 independent draws of the six-token example (one per row): every
    draw equals the oracle's, so the GPU inherits the oracle's pinned
    frequencies (0.6522 / 0.2399 / 0.1078)."""
    n = 20000
    x = np.full((n, 16), -np.inf, np.float32)
    x[:, :6] = [4.0, 3.0, 2.2, 1.6, 1.0, -2.0]
    w = dict(logits=x, dtype="f32", temperature=np.ones(n, np.float32), top_p=np.full(n, 0.9, np.float32),
             top_k=np.zeros(n, np.int32), min_p=np.zeros(n, np.float32), seed=2024, B=n, V=16)
    say("20,000 draws of the six-token example")
    tok, cnt, mk, _ = _gpu(w)
    rep, orows = oracle_and_compare(w, tok, cnt, mk)
    assert rep.ok(), rep.failures
    f = np.bincount(tok, minlength=16) / n
    assert f[3:].sum() == 0
    assert np.allclose(f[:3], [0.6522, 0.2399, 0.1078], atol=0.015)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_paths_agree_bit_for_bit(n):
    """Every path takes the same decisions with the same arithmetic: the
    split-row path, the single-workgroup path and the chunked-race path give
    identical outputs, bit for bit, including every row's probabilities."""
    import torch

    w = workloads.make(n)
    lg = device_logits(w["logits"], w["dtype"])
    say(f"workload {n}: default path")
    a = _gpu_dev(w, lg=lg, want_probs=True)
    for path in PATHS[1:]:
        say(f"workload {n}: path {path}")
        b = _gpu_dev(w, lg=lg, want_probs=True, path=path)
        for f in ("token", "keep_count", "min_kept_logit", "probs"):
            assert _same_bits(getattr(a, f), getattr(b, f)), (path, f)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_crossing_bin_overflow(dtype):
    """Rows whose crossing bin holds more tokens than the resolver's LDS list
    (one or two tied levels over 40,001 tokens; 12,000 tied tokens in ~7,600
    marked groups) or whose marked groups outnumber the list of marked groups
    (15,000 distinct values inside one bin, ~8,500 groups) are resolved by
    visiting the row in global memory; a 5,000-token crossing bin (~4,100
    marked groups) is listed from the marks; results still match the oracle
    and the single-workgroup and chunked-race paths bit for bit."""
    V = 40001
    rng = np.random.default_rng(5)
    L = np.zeros((9, V), np.float32)
    L[1, rng.random(V) < 0.5] = 1.0            # two levels, ~20K tokens each
    L[2] = rng.integers(-1, 2, V)              # three levels
    L[3, :] = 0.25                             # one level
    L[4] = rng.normal(0, 1e-6, V)              # near-constant: one narrow bin
    L[5, ::3] = -np.inf
    L[6] = rng.normal(0, 1, V)                 # 5000 tokens tied above the rest: a crossing bin
    L[6, rng.choice(V, 5000, replace=False)] = 2.5  # larger than LDS staging, within the list
    L[7] = rng.normal(0, 1, V)
    L[7, rng.choice(V, 12000, replace=False)] = 2.5  # one tied level: ~750 candidates a wave
    L[8] = rng.normal(0, 1, V)
    L[8, rng.choice(V, 15000, replace=False)] = 2.5 + rng.uniform(0, 1e-3, 15000)  # many levels in one bin
    T = np.asarray([1.0, 1.0, 0.5, 2.0, 1.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    P = np.asarray([0.5, 0.6, 0.95, 0.1, 0.5, 0.99, 0.3, 0.3, 0.4], np.float32)
    B = len(T)
    w = dict(logits=workloads.f32_to_bf16_bits(L) if dtype == "bf16" else L, dtype=dtype, temperature=T, top_p=P,
             top_k=np.zeros(B, np.int32), min_p=np.zeros(B, np.float32), seed=77, B=B, V=V)
    say(f"crossing-bin overflow rows {dtype}")
    a = _gpu(w, want_probs=True, prob_rows=range(B))
    rep, _ = oracle_and_compare(w, *a[:3], gpu_probs=a[3], prob_rows=list(range(B)))
    say(f"crossing-bin overflow {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures
    for path in ("single", "rows"):
        say(f"crossing-bin overflow {dtype}: path {path}")
        b = _gpu(w, want_probs=True, prob_rows=range(B), path=path)
        assert all(np.array_equal(np.asarray(x).view(np.uint32), np.asarray(y).view(np.uint32))
                   for x, y in zip(a, b)), path


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_logprobs_and_row_seeds(n):
    """Per-request race keys and the processed distribution's
    log-probabilities (-inf outside the nucleus) against the oracle on every
    row; every path gives the same bits."""
    import torch

    w = workloads.make(n)
    B = w["B"]
    seeds = (np.arange(B, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15) + np.uint64(12345)).astype(np.uint64)
    lg = device_logits(w["logits"], w["dtype"])
    say(f"workload {n}: per-row keys and log-probabilities, every row")
    first = _gpu_dev(w, lg=lg, want_probs=True, seeds=seeds, want_logprobs=True)
    tok, cnt, mk = _host(first)
    rep, _ = compare_every_row(w, tok, cnt, mk, probs_dev=first.probs, logprobs_dev=first.logprobs, seeds=seeds)
    say(f"workload {n} keys + logprobs: {rep.summary()}")
    assert rep.rows == B
    assert rep.ok(), rep.failures
    # The probabilities and the log-probabilities describe one distribution.
    lps, probs = first.logprobs, first.probs
    ok_rows = ~torch.isnan(lps).all(dim=1)  # (row errors are NaN throughout)
    d = (torch.exp(lps[ok_rows].double()) - probs[ok_rows].double()).abs()
    assert bool((d <= 1e-6 + 1e-5 * probs[ok_rows].double()).all())
    # The keys matter: sampled rows draw differently from the call's one seed.
    base = _host(_gpu_dev(w, lg=lg))
    sampled = (w["temperature"] > 0) & (cnt > 1)
    if sampled.sum() >= 8:
        assert (base[0][sampled] != tok[sampled]).any()
    for path in ("single", "split", "rows"):
        say(f"workload {n}: keys + logprobs on path {path}")
        other = _gpu_dev(w, lg=lg, want_probs=True, seeds=seeds, want_logprobs=True, path=path)
        for f in ("token", "keep_count", "min_kept_logit", "probs", "logprobs"):
            assert _same_bits(getattr(first, f), getattr(other, f)), (path, f)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_minp_and_greedy_row_lists(dtype):
    """Min-p and greedy rows read their tokens near the max from LDS lists
    the first pass keeps (every token at or above the first tokens' max plus
    T ln(min_p); greedy: that max), and fall back to reading the row again
    when some wave's list overflows.  Rows for both: peaked rows whose max
    lies early or late in the row; near-flat rows where most tokens are
    within T ln(1/min_p) of the max (overflow); a greedy row of one level
    (every token tied at the max: overflow) and greedy rows whose max sits in
    the last token or ties between the first and last.  Every row against
    the oracle, probabilities included, and bit for bit against the
    single-workgroup and chunked-race paths."""
    rng = np.random.default_rng(31)
    V = 65536 + 12
    rows, T, P, K, MP = [], [], [], [], []

    def add(x, t=1.0, p=0.9, k=0, mp=0.05):
        rows.append(np.asarray(x, np.float32))
        T.append(t)
        P.append(p)
        K.append(k)
        MP.append(mp)

    base = rng.normal(0, 3, V).astype(np.float32)
    add(base)                                             # list
    late = base.copy()
    late[-3] = 40.0
    add(late)                                             # max in the last tile: first max far below it
    early = base.copy()
    early[5] = 40.0
    add(early, mp=0.5)
    add(base, t=0.7, k=50)
    add(base, t=2.0, p=1.0, mp=0.01)                      # every survivor kept
    add(rng.normal(0, 0.01, V), mp=0.05)                  # near flat: overflow, row read again
    add(np.linspace(1.0, 0.0, V), t=1.0, mp=0.001)        # overflow
    add(base, t=0.0)                                      # greedy
    add(np.ones(V), t=0.0)                                # greedy, one level: overflow
    g = base.copy()
    g[-1] = 50.0
    add(g, t=-1.0)                                        # greedy, max at the last token
    g2 = base.copy()
    g2[0] = g2[-1] = 50.0
    add(g2, t=0.0)                                        # greedy tie: lowest index wins
    L = np.stack(rows)
    w = dict(logits=workloads.f32_to_bf16_bits(L) if dtype == "bf16" else L, dtype=dtype,
             temperature=np.asarray(T, np.float32), top_p=np.asarray(P, np.float32),
             top_k=np.asarray(K, np.int32), min_p=np.asarray(MP, np.float32), seed=5, B=len(T), V=V)
    B = len(T)
    say(f"min-p and greedy row lists {dtype} B={B} V={V}")
    a = _gpu(w, want_probs=True, prob_rows=range(B))
    rep, _ = oracle_and_compare(w, *a[:3], gpu_probs=a[3], prob_rows=list(range(B)))
    say(f"min-p and greedy row lists {dtype}: {rep.summary()}")
    assert rep.ok(), rep.failures
    for path in ("single", "rows"):
        b = _gpu(w, want_probs=True, prob_rows=range(B), path=path)
        assert all(np.array_equal(np.asarray(x).view(np.uint32), np.asarray(y).view(np.uint32))
                   for x, y in zip(a, b)), path
