"""Pins of the float64 oracle to things other than itself.

Each ``check_*`` function takes a loaded oracle build and raises
AssertionError when the build disagrees with what the pages or the
mathematics fix.  ``tests/test_oracle_pins.py`` runs them on the real build;
``tests/test_oracle_mutations.py`` runs them on builds with planted mistakes
and expects at least one to fail for every mistake.

The brute-force definitions below are written independently of the oracle:
no sort and no cumulative sum, just the order-free rule counted directly.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import subprocess

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _logits_of(case):
    if "logits" in case:
        return np.asarray(case["logits"], dtype=np.float32)
    spec = case["logits_spec"]
    if spec.startswith("peaked"):
        return np.asarray([8.0, 3.0, 2.0, 1.0] + [0.0] * 96, dtype=np.float32)
    if spec.startswith("sloped"):
        return np.linspace(1.0, 0.0, 100).astype(np.float32)
    raise ValueError(spec)


def run_row(O, row, T, p, k=0, mp=0.0, seed=7, step=0, probs=True):
    lg = np.asarray(row, dtype=np.float32)[None, :]
    r, pr = O.sample(lg, [T], [p], [k], [mp], seed=seed, step=step, want_probs=probs)
    return r[0], (pr[0] if probs else None)


# --------------------------------------------------------------------------
# Brute force from the definitions (independent of the oracle's code)
# --------------------------------------------------------------------------
def brute_row(x, T, p, k, mp):
    """Order-free definitions, O(V^2), no sort.

    Returns (keep mask, A (mass strictly above each token among survivors,
    normalised), probs of the kept set) for T > 0 rows with a finite logit.
    """
    x = np.asarray(x, dtype=np.float64)
    fin = x > -np.inf
    m = x[fin].max()
    e = np.where(fin, np.exp(np.where(fin, x - m, 0.0) / T), 0.0)
    prob = e / e.sum()
    surv = fin.copy()
    if mp > 0:
        surv &= ~(prob < min(mp, 1.0) * prob.max())
    if k > 0:
        greater = ((x[None, :] > x[:, None]) & surv[None, :]).sum(axis=1)
        surv &= greater < k
    q = np.where(surv, e, 0.0)
    q = q / q.sum()
    A = ((x[None, :] > x[:, None]) * q[None, :]).sum(axis=1)
    if p >= 1.0:
        keep = surv.copy()
    else:
        keep = surv & (A < p)
        top = x[surv].max()
        keep |= surv & (x == top)  # the most probable level is always kept
    ek = np.where(keep, e, 0.0)
    return keep, A, ek / ek.sum()


def exhaustive_keep(q, p):
    """Keep set by exhaustive subset search (n <= 12): take the smallest
    cardinality c of any subset whose mass reaches p (at least 1); the
    heaviest subset of that size is the top-c tokens; keep every token at
    least as probable as its lightest member (so ties share a fate)."""
    n = len(q)
    if p >= 1.0:
        return np.ones(n, bool), None
    best = None
    for c in range(1, n + 1):
        heaviest = None
        for sub in itertools.combinations(range(n), c):
            mass = sum(q[i] for i in sub)
            if heaviest is None or mass > heaviest[0]:
                heaviest = (mass, sub)
        if heaviest[0] >= p:
            best = heaviest
            break
    tau = min(q[i] for i in best[1])
    return np.asarray([qi >= tau for qi in q]), best


# --------------------------------------------------------------------------
# Checks
# --------------------------------------------------------------------------
def check_worked_examples(O):
    for case in golden()["cases"]:
        if "probs" in case:
            q = np.asarray(case["probs"], dtype=np.float64)
            keep, a, m = O.topp_levels(q, q, case["p"])
            assert keep.sum() == case["keep_count"], (case["id"], keep)
            if "renormalized" in case:
                got = q[keep] / q[keep].sum()
                assert np.allclose(got, case["renormalized"], atol=case["tol"]), (case["id"], got)
            if "kept_mass" in case:
                assert abs(q[keep].sum() - case["kept_mass"]) <= 1e-12, case["id"]
            # The same example through the full sampler, as logits ln(q).
            if case["id"] != "descending_prefix_boundary":
                r, pr = run_row(O, np.log(q).astype(np.float32), 1.0, case["p"])
                assert r["keep_count"] == case["keep_count"], (case["id"], r)
            continue
        x = _logits_of(case)
        r, pr = run_row(O, x, case["T"], case["p"])
        assert r["status"] == 0 and r["keep_count"] == case["keep_count"], (case["id"], r)
        kept = pr[pr > 0]
        if "renormalized" in case:
            got = pr[: len(case["renormalized"])]
            assert np.allclose(got, case["renormalized"], atol=case["tol"]), (case["id"], got)
            assert abs(kept.sum() - 1.0) < 1e-12
        if "kept_mass" in case:
            assert abs(r["s_keep"] / r["s_surv"] - case["kept_mass"]) <= case["tol"], (case["id"], r)
        if "tempered" in case:
            r1, p1 = run_row(O, x, case["T"], 1.0)  # p = 1: the plain tempered softmax
            assert np.allclose(p1, case["tempered"], atol=case["tempered_tol"]), (case["id"], p1)


def check_order_counterexample(O):
    """Temperature does not commute with top-p: at T = 1.5 applying top-p to
    the untempered distribution keeps 4 tokens, after temperature 5 (the
    temperature/top-k/top-p page, 'A strong answer').  The chain applies
    temperature first."""
    x = [3.0, 2.5, 2.0, 1.0, 0.5, 0.0]
    before, _ = run_row(O, x, 1.0, 0.9)
    after, pr = run_row(O, x, 1.5, 0.9)
    assert before["keep_count"] == 4 and after["keep_count"] == 5
    assert pr[4] > 0.05  # the fifth token gets a real share of the mass


def check_special_cases(O):
    # Greedy: T <= 0 is argmax with the lowest index on ties.
    r, pr = run_row(O, [1.0, 5.0, 2.0, 5.0], 0.0, 0.9)
    assert r["token"] == 1 and r["keep_count"] == 1 and pr[1] == 1.0 and pr.sum() == 1.0
    r, _ = run_row(O, [1.0, 5.0, 2.0, 5.0], -1.0, 0.9)
    assert r["token"] == 1
    # p >= 1 keeps every finite token; -inf tokens get probability 0.
    row = [0.5, -np.inf, 0.25, 3.0, -np.inf]
    r, pr = run_row(O, row, 1.0, 1.0)
    assert r["keep_count"] == 3 and pr[1] == 0.0 and pr[4] == 0.0
    r, _ = run_row(O, row, 1.0, 2.5)
    assert r["keep_count"] == 3
    # Very small and non-positive p keep the top level only (and all its ties).
    r, _ = run_row(O, [1.0, 2.0, 2.0, 0.0], 1.0, 1e-6)
    assert r["keep_count"] == 2
    r, _ = run_row(O, [1.0, 2.0, 2.0, 0.0], 1.0, 0.0)
    assert r["keep_count"] == 2
    # top_k = 1 with two equal maxima keeps both.
    r, _ = run_row(O, [4.0, 1.0, 4.0, 3.9], 1.0, 1.0, k=1)
    assert r["keep_count"] == 2
    # top_k keeps exactly k tokens when the values are distinct.
    r, _ = run_row(O, [4.0, 1.0, 3.0, 2.0], 1.0, 1.0, k=2)
    assert r["keep_count"] == 2
    # top_k >= V and top_k <= 0 are no-ops.
    for k in (0, -3, 4, 100):
        r, _ = run_row(O, [4.0, 1.0, 4.0, 3.9], 1.0, 1.0, k=k)
        assert r["keep_count"] == 4
    # min-p drops p_i < min_p * p_max; min_p > 1 behaves as 1.
    x = np.log(np.asarray([0.5, 0.25, 0.125, 0.0625, 0.0625]))
    r, _ = run_row(O, x, 1.0, 1.0, mp=0.3)
    assert r["keep_count"] == 2
    r, _ = run_row(O, x, 1.0, 1.0, mp=5.0)
    assert r["keep_count"] == 1
    # Row errors: NaN, +inf, no finite logit, NaN parameters.
    for row, T, p, mp in (([1.0, np.nan], 1.0, 0.9, 0.0), ([1.0, np.inf], 1.0, 0.9, 0.0),
                          ([-np.inf, -np.inf], 1.0, 0.9, 0.0), ([1.0, 2.0], np.nan, 0.9, 0.0),
                          ([1.0, 2.0], 1.0, np.nan, 0.0), ([1.0, 2.0], 1.0, 0.9, np.nan),
                          ([1.0, np.nan], 0.0, 0.9, 0.0)):
        r, pr = run_row(O, row, T, p, mp=mp)
        assert r["status"] == 1 and r["token"] == -1 and r["keep_count"] == 0 and not pr.any()
    # Empty batch: nothing to do, no error.
    out, _ = O.sample(np.zeros((0, 7), np.float32), np.zeros(0), np.zeros(0))
    assert out.shape == (0,)
    # -0.0 and +0.0 are one level.
    r, _ = run_row(O, [0.0, -0.0, -1.0], 1.0, 0.3)
    assert r["keep_count"] == 2


def check_bruteforce_protocol(O, batches=3000, seed=1234, extras=False):
    """Random batches of 4 rows against the order-free definition: vocabularies
    of 1 to 39 tokens, temperatures 0, 0.5, 1 and 2, p from 0.05 to 1.0, a third
    of the batches drawn from a five-value integer set so that ties are common
    (the protocol of 'Implement batched top-p sampling with temperature',
    closing paragraph of 'Why each line is there').  Tokens whose mass above
    lies within 1e-9 of p are excluded, as there.  With ``extras`` the rows
    also carry random top-k and min-p."""
    rng = np.random.default_rng(seed)
    rows_checked = boundary = 0
    for _ in range(batches):
        V = int(rng.integers(1, 40))
        if rng.random() < 1 / 3:
            L = rng.integers(-2, 3, (4, V)).astype(np.float32)
        else:
            L = rng.normal(0.0, 2.0, (4, V)).astype(np.float32)
        T = rng.choice([0.0, 0.5, 1.0, 2.0], 4).astype(np.float32)
        P = np.where(rng.random(4) < 0.1, 1.0, rng.uniform(0.05, 1.0, 4)).astype(np.float32)
        K = np.where(rng.random(4) < 0.5, rng.integers(1, V + 2, 4), 0).astype(np.int32) if extras else np.zeros(4, np.int32)
        MP = np.where(rng.random(4) < 0.5, rng.uniform(0.0, 0.6, 4), 0.0).astype(np.float32) if extras else np.zeros(4, np.float32)
        out, pr = O.sample(L, T, P, K, MP, seed=99, want_probs=True)
        for b in range(4):
            x = L[b].astype(np.float64)
            if T[b] <= 0:
                assert out[b]["token"] == int(np.argmax(x)), (L[b], out[b])
                continue
            keep, A, probs = brute_row(x, float(T[b]), float(P[b]), int(K[b]), float(MP[b]))
            near = np.abs(A - P[b]) <= 1e-9
            if P[b] < 1.0 and near.any():
                boundary += int(near.sum())
                sel = ~near
            else:
                sel = np.ones(V, bool)
            got = pr[b] > 0
            assert np.array_equal(got[sel], keep[sel]), (x, T[b], P[b], K[b], MP[b], got, keep)
            if sel.all():
                assert np.abs(pr[b] - probs).max() <= 1e-12
                assert out[b]["keep_count"] == keep.sum()
                assert keep[out[b]["token"]]
            rows_checked += 1
    return rows_checked, boundary


def check_exhaustive_subsets(O, trials=400, seed=77):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(rng.integers(1, 13))
        if rng.random() < 0.4:
            x = rng.integers(-2, 3, n).astype(np.float32)
        else:
            x = rng.normal(0.0, 1.5, n).astype(np.float32)
        p = float(rng.uniform(0.05, 1.0))
        e = np.exp(x.astype(np.float64) - x.max())
        q = e / e.sum()
        masses = [sum(q[list(s)]) for c in range(1, n + 1) for s in itertools.combinations(range(n), c)]
        if min(abs(m - p) for m in masses) <= 1e-9:
            continue  # on the boundary: floating point decides
        want, _ = exhaustive_keep(q, p)
        r, pr = run_row(O, x, 1.0, p)
        assert np.array_equal(pr > 0, want), (x, p, pr, want)


def check_invariants(O, trials=300, seed=5):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        V = int(rng.integers(2, 300))
        x = rng.normal(0, 2, V).astype(np.float32)
        if rng.random() < 0.5:
            x[rng.integers(0, V, V // 4)] = x[0]  # plant ties
        if rng.random() < 0.3:
            x[rng.integers(0, V, V // 5)] = -np.inf
            x[0] = 1.0
        T = float(rng.choice([0.3, 1.0, 2.0]))
        p = float(rng.uniform(0.05, 0.999))
        r, pr = run_row(O, x, T, p)
        keep = pr > 0
        top = x.max()
        assert keep[x == top].all()                                      # the argmax is kept
        for v in np.unique(x[np.isfinite(x)]):
            lvl = keep[x == v]
            assert lvl.all() or not lvl.any()                          # ties share a fate
        assert r["s_keep"] / r["s_surv"] >= p - 1e-12                  # kept mass reaches p
        assert abs(pr.sum() - 1.0) < 1e-12                             # renormalised
        assert not keep[~np.isfinite(x)].any()                          # -inf never kept
        assert keep[r["token"]]                                         # the draw is kept
        assert r["min_kept_logit"] == x[keep].min()
        # Temperature commutes with top-k: the kept set of top-k alone is the same at any T > 0.
        k = int(rng.integers(1, V + 1))
        a, pa = run_row(O, x, 0.5, 1.0, k=k)
        b, pb = run_row(O, x, 3.0, 1.0, k=k)
        assert np.array_equal(pa > 0, pb > 0)
        assert (pa > 0).sum() >= min(k, np.isfinite(x).sum())


def check_large_rows(O):
    """A 128,256-token row at p = 0.9 keeps far fewer than all tokens; p = 1
    keeps all of them ('Implement batched top-p sampling ...', TL;DR and
    'Why each line is there' item 3; 'Top-p (Nucleus) Sampling, in depth',
    'What to do next' item 2)."""
    V = 128256
    rng = np.random.default_rng(3)
    x = (-1.1 * np.log(rng.permutation(V) + 1.0) + rng.normal(0, 0.5, V)).astype(np.float32)
    r, _ = run_row(O, x, 1.0, 0.9, probs=False)
    assert 1 <= r["keep_count"] < V // 2
    r, _ = run_row(O, x, 1.0, 1.0, probs=False)
    assert r["keep_count"] == V


def _draw_freqs(O, case, n, seed=2024, step=0):
    x = np.asarray(case["logits"], dtype=np.float32)
    L = np.tile(x, (n, 1))
    out, _ = O.sample(L, np.full(n, case["T"]), np.full(n, case["p"]), seed=seed, step=step)
    return np.bincount(out["token"], minlength=len(x)) / n


def check_race_frequencies(O):
    """The exponential race draws from the renormalised nucleus: frequencies of
    the pages' sampled examples.  Each row of a batch has its own Philox
    counter, so a batch of n identical rows is n independent draws."""
    for case in golden()["draws"]:
        n = case["n"]
        f = _draw_freqs(O, case, n)
        k = len(case["target"])
        assert f[k:].sum() == 0.0, f                       # nothing outside the nucleus
        for got, want in zip(f[:k], case["target"]):
            sigma = math.sqrt(want * (1 - want) / n)
            assert abs(got - want) <= 5 * sigma + 1e-3, (case["id"], f)


def check_race_chisquare(O):
    """400,000 draws from a filtered 5-token distribution: chi-square at a fixed
    seed, and no filtered-out token ever drawn ('Implement batched top-p
    sampling ...', closing paragraph of 'Why each line is there')."""
    q = np.asarray([0.30, 0.25, 0.25, 0.12, 0.08])
    x = np.log(q).astype(np.float32)
    n = 400_000
    out, pr = O.sample(np.tile(x, (n, 1)), np.ones(n), np.full(n, 0.6), seed=31337, step=5)
    target = np.asarray([0.375, 0.3125, 0.3125, 0.0, 0.0])
    cnt = np.bincount(out["token"], minlength=5)
    assert cnt[3] == 0 and cnt[4] == 0
    exp = target[:3] * n
    chi2 = float(((cnt[:3] - exp) ** 2 / exp).sum())
    assert chi2 < 18.4, (cnt, chi2)  # chi-square with 2 dof: p-value 1e-4
    tv = 0.5 * np.abs(cnt / n - target).sum()
    assert tv < 0.005, tv


def check_race_reproducible(O):
    x = np.random.default_rng(8).normal(0, 1, (64, 500)).astype(np.float32)
    T = np.ones(64, np.float32)
    P = np.full(64, 0.95, np.float32)
    a, _ = O.sample(x, T, P, seed=11, step=3)
    b, _ = O.sample(x, T, P, seed=11, step=3)
    c, _ = O.sample(x, T, P, seed=11, step=4)
    d, _ = O.sample(x, T, P, seed=12, step=3)
    assert np.array_equal(a["token"], b["token"])
    assert (a["token"] != c["token"]).sum() > 32
    assert (a["token"] != d["token"]).sum() > 32


_ROCRAND_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "rocrand_philox_words.cpp")


def rocrand_words(tuples, workdir):
    """Philox4x32-10 words from rocRAND's engine (host build) for
    (seed, step, row, token) tuples."""
    exe = os.path.join(workdir, "rocrand_philox_words")
    if not os.path.exists(exe):
        subprocess.run(["hipcc", "-O1", "--offload-arch=gfx950", "-o", exe, _ROCRAND_SRC], check=True,
                       cwd=workdir)
    text = "".join(f"{s} {t} {r} {i}\n" for s, t, r, i in tuples)
    res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    return [int(v) for v in res.stdout.split()]


def philox_tuples(n=3000, seed=9):
    rng = np.random.default_rng(seed)
    # rocRAND addresses words by a 64-bit offset = 4 * counter(words 0,1), so the
    # row (counter word 1) stays below 2**30 here.
    tuples = [(0, 0, 0, 0), (1, 0, 0, 0), (2**64 - 1, 2**64 - 1, 2**30 - 1, 2**31 - 1)]
    for _ in range(n):
        tuples.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)), int(rng.integers(0, 2**63)),
                       int(rng.integers(0, 2**30)), int(rng.integers(0, 2**31))))
    return tuples


def check_philox_against(O, tuples, words):
    for (s, t, r, i), w in zip(tuples, words):
        assert O.noise_word(s, t, r, i) == w, (s, t, r, i)


def check_exp1(O):
    """u = (r + 1/2)/2^32 and E = -ln u, at the extremes and midpoint."""
    assert abs(O.exp1(0) - (-math.log(0.5 / 2**32))) < 1e-12
    assert abs(O.exp1(2**32 - 1) - (-math.log1p(-0.5 / 2**32))) < 1e-20
    assert abs(O.exp1(2**31) - (-math.log((2**31 + 0.5) / 2**32))) < 1e-15


def check_logprobs(O):
    """Processed-distribution log-probabilities: ln p_i on the kept set, -inf
    outside it (outside the nucleus the probability is zero), NaN on error
    rows.  Pinned to the printed worked examples, a closed form, a kept token
    whose weight underflows, and invariants on random rows."""
    for case in golden()["cases"]:
        if "probs" in case or "renormalized" not in case:
            continue
        x = _logits_of(case)
        r, pr, lp = O.sample(x[None, :], [case["T"]], [case["p"]], want_probs=True, want_logprobs=True)
        n = len(case["renormalized"])
        assert np.allclose(np.exp(lp[0, :n]), case["renormalized"], atol=case["tol"]), (case["id"], lp[0, :n])
        assert np.all(np.isneginf(lp[0][pr[0] == 0])), case["id"]
    # T = +inf: every finite token weighs the same, ln p = -ln(n finite).
    x = np.array([[0.5, -2.0, 3.0, -np.inf, 1.0]], dtype=np.float32)
    r, pr, lp = O.sample(x, [np.inf], [1.0], want_probs=True, want_logprobs=True)
    assert np.allclose(lp[0, [0, 1, 2, 4]], -math.log(4.0), atol=1e-15) and np.isneginf(lp[0, 3])
    # p = 1 keeps a token of weight e^-800 (it underflows in double); its
    # log-probability is -800 - ln(1 + e^-800) = -800.
    r, pr, lp = O.sample(np.array([[0.0, -800.0]], dtype=np.float32), [1.0], [1.0], want_probs=True,
                         want_logprobs=True)
    assert pr[0, 1] == 0.0 and lp[0, 1] == -800.0 and lp[0, 0] == 0.0
    # Greedy: 0 at the lowest-index max, -inf elsewhere; an error row is NaN.
    r, pr, lp = O.sample(np.array([[1.0, 3.0, 3.0, 2.0], [1.0, np.nan, 0.0, 0.0]], dtype=np.float32),
                         [0.0, 1.0], [0.9, 0.9], want_probs=True, want_logprobs=True)
    assert lp[0, 1] == 0.0 and np.all(np.isneginf(lp[0, [0, 2, 3]])) and np.all(np.isnan(lp[1]))
    # Random rows at several temperatures: the kept log-probabilities sum to one
    # in the exponential and differ by (x_i - x_j)/T.
    rng = np.random.default_rng(12)
    for T in (0.3, 1.0, 2.5):
        x = rng.normal(0.0, 2.0, (4, 200)).astype(np.float32)
        r, pr, lp = O.sample(x, [T] * 4, [0.9] * 4, want_probs=True, want_logprobs=True)
        for b in range(4):
            k = pr[b] > 0
            assert abs(np.exp(lp[b][k]).sum() - 1.0) < 1e-12
            i, j = np.flatnonzero(k)[:2] if k.sum() > 1 else (np.flatnonzero(k)[0],) * 2
            T32 = float(np.float32(T))  # the oracle takes T as float32
            assert abs((lp[b, i] - lp[b, j]) - (float(x[b, i]) - float(x[b, j])) / T32) < 1e-12


def check_row_seeds(O):
    """Per-request race keys: row b with key seeds[b] draws what a call with
    seed = seeds[b] draws for it, whatever the other rows' keys."""
    rng = np.random.default_rng(3)
    B, V = 6, 60
    x = rng.normal(0.0, 1.0, (B, V)).astype(np.float32)
    T, P = [1.0] * B, [0.95] * B
    seeds = np.arange(100, 100 + B, dtype=np.uint64)
    a, _ = O.sample(x, T, P, seed=0, step=3, seeds=seeds)
    for b in range(B):
        one, _ = O.sample(x, T, P, seed=int(seeds[b]), step=3, rows=[b])
        assert one["token"][b] == a["token"][b], b
    other = seeds.copy()
    other[1:] += 1000
    c, _ = O.sample(x, T, P, seed=0, step=3, seeds=other)
    assert c["token"][0] == a["token"][0]
    # The keys matter: 40 flat rows with distinct keys do not all draw what one
    # common key draws.
    flat = np.zeros((40, 30), dtype=np.float32)
    d, _ = O.sample(flat, [1.0] * 40, [1.0] * 40, seed=5, step=0)
    e, _ = O.sample(flat, [1.0] * 40, [1.0] * 40, seed=5, step=0, seeds=np.arange(40, dtype=np.uint64) + 9)
    assert (d["token"] != e["token"]).any()




# --------------------------------------------------------------------------
# The rejection sampler ("Top-p (Nucleus) Sampling, in depth", "Sort-free
# top-p by rejection sampling")
# --------------------------------------------------------------------------
def rejection_exact(x, T, p, mp):
    """Exact law of the pivot process on a tiny row, by recursion over pivots
    (independent of the oracle): a proposal is drawn proportionally to e among
    the finite tokens above the pivot; it is accepted iff it survives min-p and
    is in the top level or its survivor mass strictly above is < p S;
    otherwise the pivot moves to it.  Returns (accepted-token distribution,
    expected rounds, expected squared rounds)."""
    x = np.asarray(x, dtype=np.float64)
    fin = x > -np.inf
    m = x[fin].max()
    e = np.where(fin, np.exp(np.where(fin, x - m, 0.0) / T), 0.0)
    surv = fin & ~(e < min(mp, 1.0)) if mp > 0 else fin.copy()
    S = e[surv].sum()

    def accepted(t):
        if not surv[t]:
            return False
        if x[t] == m:
            return True
        return p > 0 and e[surv & (x > x[t])].sum() < p * S

    memo = {}

    def go(pivot):
        if pivot in memo:
            return memo[pivot]
        props = np.nonzero(fin & (x > pivot))[0]
        W = e[props].sum()
        dist = np.zeros(len(x))
        r1, r2 = 1.0, 1.0
        for t in props:
            q = e[t] / W
            if accepted(t):
                dist[t] += q
            else:
                d, a1, a2 = go(float(x[t]))
                dist += q * d
                r1 += q * a1          # rounds = 1 + R'
                r2 += q * (2 * a1 + a2)  # E[(1 + R')^2] - 1 over this branch
        memo[pivot] = (dist, r1, r2)
        return memo[pivot]

    return go(-np.inf)


def check_rejection_pages(O):
    """The pages' rejection run: 40,000 draws of the six-token example at
    p = 0.9 land on the renormalised nucleus and take about 1.09 rounds."""
    for case in golden()["rejection"]:
        x = np.asarray(case["logits"], dtype=np.float32)
        n, k = case["n"], len(case["target"])
        dist, r1, r2 = rejection_exact(x, case["T"], case["p"], 0.0)
        # The exact law is the renormalised nucleus the pages print.
        assert np.abs(dist[:k] - case["target"]).max() < 5e-5 and dist[k:].sum() == 0.0, dist
        assert abs(r1 - case["printed_rounds_mean"]) < 0.005, r1
        for got, want in zip(case["printed_freqs"], case["target"]):
            assert abs(got - want) <= 5 * math.sqrt(want * (1 - want) / n) + 1e-3
        out = O.sample_rejection(np.tile(x, (n, 1)), np.full(n, case["T"]), np.full(n, case["p"]),
                                 seed=2024, step=0)
        assert (out["status"] == 0).all()
        f = np.bincount(out["token"], minlength=len(x)) / n
        assert f[k:].sum() == 0.0, f
        for got, want in zip(f[:k], dist[:k]):
            assert abs(got - want) <= 5 * math.sqrt(want * (1 - want) / n) + 1e-3, (f, dist)
        sd = math.sqrt(max(r2 - r1 * r1, 0.0))
        assert abs(out["rounds"].mean() - r1) <= 5 * sd / math.sqrt(n) + 1e-3, (out["rounds"].mean(), r1)


def check_rejection_law(O, cases=24, n=12000, seed=91):
    """Tiny random rows (ties, -inf padding, min-p, p <= 0, p >= 1): the
    oracle's accepted-token frequencies and mean rounds match the exact law of
    the pivot process, and that law is the renormalised kept distribution of
    the brute-force definition."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        V = int(rng.integers(2, 8))
        x = rng.normal(0, 1.5, V)
        if c % 3 == 0:
            x = np.round(x * 2) / 2            # ties
        if c % 5 == 0:
            x[rng.integers(0, V)] = -np.inf    # a masked token
            if not np.isfinite(x).any():
                x[0] = 0.0
        x = x.astype(np.float32)
        T = float(np.float32(rng.uniform(0.4, 2.0)))
        p = [0.0, 1.0, float(np.float32(rng.uniform(0.05, 0.99)))][c % 3 if c % 4 else 2]
        mp = float(np.float32(rng.uniform(0.01, 0.4))) if c % 4 == 1 else 0.0
        dist, r1, r2 = rejection_exact(x, T, p, mp)
        keep, _, probs = brute_row(x, T, p, 0, mp)
        assert np.allclose(dist, probs, atol=1e-12), (x, T, p, mp, dist, probs)
        out = O.sample_rejection(np.tile(x, (n, 1)), np.full(n, T), np.full(n, p),
                                 min_p=np.full(n, mp), seed=1000 + c, step=3)
        assert (out["status"] == 0).all() and (out["rounds"] >= 1).all()
        f = np.bincount(out["token"], minlength=V) / n
        assert f[~keep].sum() == 0.0, (f, keep)
        for got, want in zip(f, dist):
            assert abs(got - want) <= 5 * math.sqrt(max(want * (1 - want), 0.0) / n) + 1e-3, (c, f, dist)
        sd = math.sqrt(max(r2 - r1 * r1, 0.0))
        assert abs(out["rounds"].mean() - r1) <= 5 * sd / math.sqrt(n) + 1e-3, (c, out["rounds"].mean(), r1)
        levels = len(np.unique(x[np.isfinite(x)]))
        assert out["rounds"].max() <= levels


def check_rejection_is_the_race(O, B=200, V=400, seed=17):
    """With the row's own noise words in every round, the accepted token is
    the first kept token in race order: the main sampler's token, unless the
    row sits on a boundary (mass within 1e-12 of p, or a race tie).  Greedy
    and error rows follow the main sampler's rules with 0 rounds."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 2, (B, V))
    x[::3] = np.round(x[::3] * 4) / 4
    x[1::7, : V // 3] = -np.inf
    x = x.astype(np.float32)
    T = rng.uniform(0.3, 2.0, B).astype(np.float32)
    T[::11] = 0.0
    P = rng.uniform(0.0, 1.0, B).astype(np.float32)
    P[::13] = 1.0
    P[5::13] = 0.0
    MP = np.where(rng.random(B) < 0.3, rng.uniform(0.001, 0.3, B), 0.0).astype(np.float32)
    P[13::26] = 1.5   # p > 1 acts as p = 1
    MP[13::26] = 0.2  # with min-p: most proposals then fail min-p alone
    x[7, 3] = np.nan
    P[9] = np.nan
    ref, _ = O.sample(x, T, P, None, MP, seed=99, step=4)
    out = O.sample_rejection(x, T, P, MP, seed=99, step=4)
    for b in range(B):
        if ref["status"][b]:
            assert out["status"][b] == 1 and out["token"][b] == -1 and out["rounds"][b] == 0
            continue
        if T[b] <= 0:
            assert out["greedy"][b] == 1 and out["rounds"][b] == 0 and out["token"][b] == ref["token"][b]
            continue
        assert out["status"][b] == 0 and out["rounds"][b] >= 1
        if out["band"][b] > 1e-12 and out["race_margin"][b] > 1e-12:
            assert out["token"][b] == ref["token"][b], b
        if P[b] >= 1.0 and MP[b] == 0.0:
            assert out["rounds"][b] == 1  # every finite token is kept
    assert (out["rounds"][T > 0] > 1).any()  # some rows did reject




# --------------------------------------------------------------------------
# Speculative acceptance ("Top-p (Nucleus) Sampling, in depth", "Logprobs,
# speculative decoding and reproducibility")
# --------------------------------------------------------------------------
def _spec_draws(O, x, T, p, k, mp, q, n, seed, step=0):
    """n independent verifications of one row (each batch row has its own
    Philox counter) with draft tokens drawn from q by NumPy."""
    V = len(x)
    qq = np.asarray(q, np.float32).astype(np.float64)
    d = np.random.default_rng(seed).choice(V, size=n, p=qq / qq.sum())
    out = O.spec_verify(np.tile(x, (n, 1)), np.full(n, T), np.full(n, p), np.full(n, k, np.int32), np.full(n, mp),
                        np.tile(np.asarray(q, np.float32), (n, 1)), d, seed=seed, step=step)
    return out, d


def check_spec_law(O, cases=20, n=12000, seed=404):
    """Whatever the draft q, the verified token follows the truncated target
    p exactly (brute-force definition), the acceptance rate is
    sum_i min(p_i, q_i), and no token outside the nucleus is ever output;
    the pages' six-token example included."""
    rng = np.random.default_rng(seed)
    spec = golden()["speculative"]
    for c in range(cases + len(spec)):
        if c < len(spec):
            case = spec[c]
            x = np.asarray(case["logits"], np.float32)
            T, p, k, mp = case["T"], case["p"], 0, 0.0
            qx = np.exp(x.astype(np.float64) + np.asarray(case["draft_logit_shift"]))
            nn = case["n"]
        else:
            V = int(rng.integers(2, 8))
            x = rng.normal(0, 1.5, V)
            if c % 3 == 0:
                x = np.round(x * 2) / 2
            x = x.astype(np.float32)
            T = float(np.float32(rng.uniform(0.5, 2.0)))
            p = float(np.float32(rng.uniform(0.2, 1.0)))
            k = int(rng.integers(0, V + 1)) if c % 4 == 1 else 0
            mp = float(np.float32(rng.uniform(0.01, 0.3))) if c % 5 == 2 else 0.0
            qx = np.exp(rng.normal(0, 1.0, V))
            if c % 3 == 1:
                qx[rng.integers(0, V)] = 0.0  # the draft never proposes this token
            nn = n
        q = (qx / qx.sum()).astype(np.float32)
        keep, _, target = brute_row(x, T, p, k, mp)
        if c < len(spec):
            assert np.abs(target[: len(spec[c]["target"])] - spec[c]["target"]).max() < 5e-5
        out, d = _spec_draws(O, x, T, p, k, mp, q, nn, seed=1000 + c)
        assert (out["status"] == 0).all()
        f = np.bincount(out["token"], minlength=len(x)) / nn
        assert f[~keep].sum() == 0.0, (c, f, keep)
        for got, want in zip(f, target):
            assert abs(got - want) <= 5 * math.sqrt(max(want * (1 - want), 0.0) / nn) + 1e-3, (c, f, target)
        rate = float(np.minimum(target, q.astype(np.float64)).sum())
        assert abs(out["accepted"].mean() - rate) <= 5 * math.sqrt(rate * (1 - rate) / nn) + 1e-3, (c, rate)
        acc = out["accepted"] == 1
        assert (out["token"][acc] == d[acc]).all()


def check_spec_special(O):
    """q = p accepts every draft; a draft that proposes only a token outside
    the nucleus is never accepted and the output then follows p; a target
    row error or a draft token out of range is a row error."""
    x = np.asarray([2.0, 1.0, 0.5, -1.0, -3.0], np.float32)
    keep, _, target = brute_row(x, 1.0, 0.8, 0, 0.0)
    n = 20000
    out, _ = _spec_draws(O, x, 1.0, 0.8, 0, 0.0, target, n, seed=1)
    assert out["accepted"].mean() > 0.999
    outside = int(np.nonzero(~keep)[0][0])
    q = np.zeros(len(x))
    q[outside] = 1.0
    out, d = _spec_draws(O, x, 1.0, 0.8, 0, 0.0, q, n, seed=2)
    assert (d == outside).all() and out["accepted"].sum() == 0
    f = np.bincount(out["token"], minlength=len(x)) / n
    for got, want in zip(f, target):
        assert abs(got - want) <= 5 * math.sqrt(max(want * (1 - want), 0.0) / n) + 1e-3
    bad = np.tile(x, (3, 1))
    bad[0, 1] = np.nan
    out = O.spec_verify(bad, np.ones(3), np.full(3, 0.8), None, None, np.full((3, 5), 0.2, np.float32),
                        np.asarray([0, 5, -1]), seed=3)
    assert (out["status"] == 1).all() and (out["token"] == -1).all()




# --------------------------------------------------------------------------
# The pre-chain: penalties and the grammar mask ("Top-p (Nucleus) Sampling,
# in depth", "Where top-p sits in the sampler chain"; "What do temperature,
# top-k and top-p ...", "What interviewers probe next")
# --------------------------------------------------------------------------
def check_preprocess_values(O):
    """Values worked by hand from the definitions: repetition 2, frequency
    0.25, presence 0.5; history [0, 1, 1, 3]; token 4 disallowed.
      token 0: x = 2 > 0 -> 2 / 2 = 1; minus 0.25 * 1 + 0.5 -> 0.25
      token 1: x = -1 -> -1 * 2 = -2; seen twice: minus 0.25 * 2 + 0.5 -> -3
      token 3: x = 3 -> 1.5; minus 0.75 -> 0.75
      tokens 2 and 5 are not in the history; token 4 is masked."""
    x = np.asarray([[2.0, -1.0, 0.5, 3.0, -2.0, 1.0]], np.float32)
    out = O.preprocess(x, hist=np.asarray([[0, 1, 1, 3, -1, 17]]), repetition=[2.0], frequency=[0.25],
                       presence=[0.5], allowed=np.asarray([[0b101111]], np.uint32))
    assert np.array_equal(out, np.asarray([[0.25, -3.0, 0.5, 0.75, -np.inf, 1.0]], np.float32)), out
    # Bit i of word i / 32: token 33 is bit 1 of the second word.
    x = np.zeros((1, 40), np.float32)
    m = np.asarray([[0xFFFFFFFF, 0xFFFFFFFD]], np.uint32)
    out = O.preprocess(x, allowed=m)
    assert np.isneginf(out[0, 33]) and np.isfinite(out[0, np.arange(40) != 33]).all()


def check_preprocess_identity_and_invariants(O, seed=12):
    """No penalty and no mask changes nothing, bit for bit (bf16 widened
    exactly); tokens outside the history keep their logits; with rho >= 1 and
    non-negative a_f, a_p a history token never rises."""
    rng = np.random.default_rng(seed)
    B, V, H = 6, 300, 40
    x = rng.normal(0, 3, (B, V)).astype(np.float32)
    hist = rng.integers(-1, V, (B, H)).astype(np.int32)
    out = O.preprocess(x, hist=hist, repetition=np.ones(B), frequency=np.zeros(B), presence=np.zeros(B))
    assert np.array_equal(out.view(np.uint32), x.view(np.uint32))
    import workloads
    xb = workloads.f32_to_bf16_bits(x)
    assert np.array_equal(O.preprocess(xb), workloads.bf16_bits_to_f32(xb))
    rep = rng.uniform(1.0, 2.0, B).astype(np.float32)
    fr = rng.uniform(0, 1, B).astype(np.float32)
    pr = rng.uniform(0, 1, B).astype(np.float32)
    out = O.preprocess(x, hist=hist, repetition=rep, frequency=fr, presence=pr)
    for b in range(B):
        seen = np.zeros(V, bool)
        seen[hist[b][hist[b] >= 0]] = True
        assert np.array_equal(out[b, ~seen], x[b, ~seen])
        assert (out[b, seen] <= x[b, seen]).all()
        # Presence alone lowers every seen token by exactly a_p (where that is exact).
    one = O.preprocess(x[:1], hist=np.asarray([[5, 5, 5]]), frequency=[0.5])
    assert one[0, 5] == np.float32(x[0, 5] - np.float32(1.5))


def check_chain_order(O):
    """Masks come before top-p: a nucleus never holds a forbidden token, even
    when the forbidden tokens carry most of the mass ("Where top-p sits in the
    sampler chain").  Repetition penalties act on raw logits and change the
    greedy choice too ("What interviewers probe next")."""
    x = np.asarray([[5.0, 4.8, 1.0, 0.9, 0.5, 0.2, 0.1, 0.0]], np.float32)
    allowed = np.asarray([[0b11111100]], np.uint32)  # the two heavy tokens are forbidden
    xp = O.preprocess(x, allowed=allowed)
    n = 4000
    out, _ = O.sample(np.tile(xp, (n, 1)), np.ones(n), np.full(n, 0.5), seed=8)
    assert (out["status"] == 0).all() and (out["token"] >= 2).all()
    assert (out["keep_count"] >= 1).all()
    raw, _ = O.sample(np.tile(x, (n, 1)), np.ones(n), np.full(n, 0.5), seed=8)
    assert (raw["token"] < 2).all()  # the same chain without the mask keeps only forbidden tokens
    g = np.asarray([[3.0, 2.5, 1.0]], np.float32)
    gp = O.preprocess(g, hist=np.asarray([[0]]), repetition=[2.0])
    assert O.sample(g, [0.0], [1.0])[0]["token"][0] == 0
    assert O.sample(gp, [0.0], [1.0])[0]["token"][0] == 1


# --------------------------------------------------------------------------
# The judges of boundary rows: oracle_eval_cut and oracle_race_score
# --------------------------------------------------------------------------
def _levels_numpy(x, T, k, mp):
    """Survivor levels of a row from the definitions with numpy's sort:
    (survivor mask, weights e, sorted distinct survivor values descending,
    mass strictly above each of them, mass at each), masses normalised over
    the survivors ("Implement batched top-p sampling with temperature", "How
    to approach it": a token's mass above is that of every strictly more
    probable token; "What do temperature, top-k and top-p each do ...",
    reference sampler: min-p and top-k cut the tempered distribution)."""
    x = np.asarray(x, dtype=np.float64)
    fin = x > -np.inf
    m = x[fin].max()
    e = np.where(fin, np.exp(np.where(fin, x - m, 0.0) / T), 0.0)
    surv = fin.copy()
    if mp > 0:
        surv &= ~(e < min(mp, 1.0))  # p_i < min_p p_max, with p_max the weight 1 of the max
    if k > 0:
        vals = np.sort(x[surv])[::-1]
        if k < vals.size:
            surv &= x >= vals[k - 1]
    S = e[surv].sum()
    lv, inv = np.unique(x[surv], return_inverse=True)
    at = np.bincount(inv, weights=e[surv] / S, minlength=lv.size)[::-1]
    lv = lv[::-1]
    above = np.concatenate([[0.0], np.cumsum(at)[:-1]])
    return surv, e, lv, above, at


def _race_score_numpy(O, x, row, T, seed, step, tok):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp((x[tok] - x[x > -np.inf].max()) / T)
    E = -np.log((O.noise_word(seed, step, row, tok) + 0.5) * 2.0 ** -32)
    return e / E


def check_judges(O, batches=150, seed=31):
    """oracle_eval_cut and oracle_race_score against the definitions.  They
    judge the rows within 1e-5 of a mass boundary, where the pages say the
    keep rule itself is ambiguous under floating point ("Implement batched
    top-p ...", "Why each line is there", closing paragraph), so they get pins
    of their own.  Per non-greedy row (tiny random rows with and without
    min-p/top-k, and rows of the small and tie-heavy workloads):
    - at the oracle's own smallest kept logit, eval_cut gives the oracle's
      keep count, token and winning score, and (A, M) of that level as
      computed here (to 1e-13 + 1e-15 V: the same masses summed in another
      order); at the survivor levels just above and below, and at a
      value below every survivor, the masses of those levels and the count
      of survivors at or above them, and (1, 1) with every survivor kept
      below the lowest survivor and below every finite logit;
    - race_score of the drawn token is e/E written out from the token's
      noise word, and equals the oracle's winning score."""
    import workloads

    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(batches):
        V = int(rng.integers(1, 40))
        L = (rng.integers(-2, 3, (4, V)) if rng.random() < 1 / 3 else rng.normal(0, 2, (4, V))).astype(np.float32)
        if rng.random() < 0.3:
            L[:, rng.random(V) < 0.2] = -np.inf
            L[:, 0] = 0.5
        T = rng.choice([0.5, 1.0, 2.0], 4).astype(np.float32)
        P = np.where(rng.random(4) < 0.1, 1.0, rng.uniform(0.05, 1.0, 4)).astype(np.float32)
        K = np.where(rng.random(4) < 0.5, rng.integers(1, V + 2, 4), 0).astype(np.int32)
        MP = np.where(rng.random(4) < 0.5, rng.uniform(0.0, 0.6, 4), 0.0).astype(np.float32)
        cases.append((L, T, P, K, MP, 99))
    for n, rows in ((1, None), (2, range(6))):
        w = workloads.make(n, rows=rows)
        cases.append((w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], w["seed"]))
    checked = 0
    for L, T, P, K, MP, sd in cases:
        out, _ = O.sample(L, T, P, K, MP, seed=sd)
        for b in range(L.shape[0]):
            o = out[b]
            if o["status"] != 0 or o["greedy"]:
                continue
            x = L[b].astype(np.float64)
            tol = 1e-13 + 1e-15 * x.size  # two summation orders of the same masses
            surv, e, lv, above, at = _levels_numpy(x, float(T[b]), int(K[b]), float(MP[b]))
            cut = float(o["min_kept_logit"])
            ev, _ = O.eval_cut(L[b], b, T[b], P[b], K[b], MP[b], sd, 0, cut)
            j = int(np.nonzero(lv == cut)[0][0])
            assert ev["status"] == 0
            assert ev["keep_count"] == o["keep_count"] == int((surv & (x >= cut)).sum())
            assert ev["token"] == o["token"]
            assert abs(ev["race_s1"] - o["race_s1"]) <= 1e-12 * o["race_s1"]
            assert abs(ev["a_cut"] - above[j]) <= tol and abs(ev["m_cut"] - (above[j] + at[j])) <= tol
            if o["topp_active"]:
                assert abs(ev["a_cut"] - o["a_star"]) <= tol and abs(ev["m_cut"] - o["m_star"]) <= tol
            for jj in (j - 1, j + 1):
                if 0 <= jj < lv.size:
                    en, _ = O.eval_cut(L[b], b, T[b], P[b], K[b], MP[b], sd, 0, float(lv[jj]))
                    assert abs(en["a_cut"] - above[jj]) <= tol
                    assert abs(en["m_cut"] - (above[jj] + at[jj])) <= tol
                    assert en["keep_count"] == int((surv & (x >= lv[jj])).sum())
            # Just below the lowest survivor, and below every finite logit
            # (where min-p or top-k leave non-survivors): every survivor is
            # above, nothing else counts.
            for low in (float(np.nextafter(np.float32(lv[-1]), np.float32(-np.inf))), -3.4028234663852886e38):
                if low > -np.inf:
                    en, _ = O.eval_cut(L[b], b, T[b], P[b], K[b], MP[b], sd, 0, low)
                    assert abs(en["a_cut"] - 1.0) <= tol and abs(en["m_cut"] - 1.0) <= tol
                    assert en["keep_count"] == int(surv.sum())
            sc = O.race_score(L[b], b, T[b], sd, 0, int(o["token"]))
            want = _race_score_numpy(O, x, b, float(T[b]), sd, 0, int(o["token"]))
            assert abs(sc - want) <= 1e-12 * want and abs(sc - o["race_s1"]) <= 1e-12 * want
            checked += 1
    assert checked > 400
    return checked


ALL_FAST_CHECKS = [check_worked_examples, check_order_counterexample, check_special_cases, check_invariants,
                   check_exp1, check_race_reproducible, check_logprobs, check_row_seeds, check_rejection_pages,
                   check_rejection_law, check_rejection_is_the_race, check_spec_law, check_spec_special,
                   check_preprocess_values, check_preprocess_identity_and_invariants, check_chain_order,
                   check_judges]
