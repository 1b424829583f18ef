"""Rows built on the host where the exponential race is decided by a hair.

The race draws token argmax_i e_i / E_i with E_i = -ln u_i from the token's
Philox word ("What do temperature, top-k and top-p each do ...", "A strong
answer", last paragraph: the race draws exactly from p).  Fast race code
screens tokens against the best score seen so far with a bound on E that is
tight when 1 - u sits just above a power of two; a margin on the wrong side of
that bound drops a winner that beats the running best by a fraction of a
percent.  These rows put exactly that case in front of every path:

- a max token (logit 0, weight 1) whose E is the row's largest, so its score
  1/E1 is small;
- every other token (the runner-ups) with a logit chosen so that its score is
  1/E1 times (1 - delta), delta in [1e-5, 5e-5]: whatever token a lane races
  first, its running best ends within 5e-5 of 1/E1;
- one winner whose word w has ~w in [2^k, 2^k (1 + 2^-9)] for some
  k <= 22 (1 - u just above a power of two, and small, so E is close to
  1 - u), placed away from the start of the row, its chunk and its item, with
  a logit that makes its score 1/E1 times (1 + 2e-5).

The noise words come from the oracle (oracle.noise_words); the logits are
chosen in float64 from the oracle's E and rounded to float32 once.  The
builder then asks the oracle which token wins and keeps only rows where that
is the planted winner with a race margin above 1e-6 (so no exemption applies).
"""
from __future__ import annotations

import numpy as np

DELTA_WIN = 2e-5
DELTA_LO, DELTA_HI = 1e-5, 5e-5


def _winner_candidates(words: np.ndarray, V: int) -> np.ndarray:
    n = (~words).astype(np.uint64)  # 2^32 - 1 - word: 1 - u in units of 2^-32 (minus one half)
    idx = np.arange(V)
    ok = (n >= 64) & (n < (1 << 23))
    k = np.floor(np.log2(np.maximum(n, 1).astype(np.float64))).astype(np.int64)
    frac = n.astype(np.float64) / np.exp2(k) - 1.0
    ok &= frac <= 2.0 ** -9
    # Away from the row's start, from the start of an 8192-token chunk and of
    # a 2048-token item (where a lane might race it before any runner-up).
    ok &= (idx >= V // 4) & ((idx % 8192) >= 1024) & ((idx % 2048) >= 512)
    return idx[ok]


def build(orc, B: int, V: int, base_seed: int, step: int = 0, temps=(1.0, 0.7, 1.3)):
    """Returns (logits [B, V] f32, T [B], seeds [B] u64, winners [B]).  Row b
    races under its own key seeds[b] (the per-request key option), the first
    key from base_seed + 4096 b on whose noise has a winner candidate."""
    rng = np.random.default_rng(base_seed ^ 0x5A5A)
    logits = np.empty((B, V), np.float32)
    T = np.empty(B, np.float32)
    seeds = np.empty(B, np.uint64)
    winners = np.empty(B, np.int64)
    for b in range(B):
        for t in range(4096):
            sd = base_seed + 4096 * b + t
            words = orc.noise_words(sd, step, b, V)
            cands = _winner_candidates(words, V)
            if cands.size:
                break
        else:
            raise RuntimeError(f"row {b}: no winner candidate in 4096 keys")
        i2 = int(cands[rng.integers(0, cands.size)])
        E = -np.log((words.astype(np.float64) + 0.5) * 2.0 ** -32)
        Ew = E.copy()
        Ew[i2] = -np.inf
        i1 = int(np.argmax(Ew))
        s1 = 1.0 / E[i1]
        tt = float(temps[b % len(temps)])
        delta = rng.uniform(DELTA_LO, DELTA_HI, V)
        e = s1 * (1.0 - delta) * E
        e[i1] = 1.0
        e[i2] = s1 * (1.0 + DELTA_WIN) * E[i2]
        x = tt * np.log(e)
        x[(e >= 0.999) & (np.arange(V) != i1)] = -np.inf
        x[i1] = 0.0
        logits[b] = x.astype(np.float32)
        T[b] = tt
        seeds[b] = sd
        winners[b] = i2
    return logits, T, seeds, winners


def screen_rejects(x_win: float, m: float, T: float, sstar: float, word: int, margin: float) -> bool:
    """The race screen's test, in float32 as the kernels evaluate it: True if
    a token of logit x_win and noise word `word` is screened out against a
    running best `sstar` with R = (x - m) c - log2 sstar + margin.  fma is
    emulated exactly in float64 and rounded once."""
    f32 = np.float32
    n = f32(np.uint32(~np.uint32(word)))  # ~word as a float (round to nearest)
    bits = float(f32(np.float32(n).view(np.uint32)))
    L = f32(bits * 2.0 ** -23 + float(f32(-159.00005)))
    c = f32(f32(1.0) / f32(T)) * f32(1.4426950408889634)
    q = f32(-f32(np.log2(f32(sstar)))) + f32(margin)
    d = f32(f32(x_win) - f32(m))
    R = f32(float(d) * float(c) + float(q))
    return bool(L > R)


def build_rejection(orc, B: int, V: int, base_seed: int, step: int = 0):
    """Rows for the rejection sampler's proposal chain ("Top-p (Nucleus)
    Sampling, in depth", "Sort-free top-p by rejection sampling"), T = 1.

    Round 1 races every finite token; its winner W1 (the token with the
    smallest E, given a tiny weight) lies outside the nucleus and becomes the
    pivot.  Round 2's proposal is the best score above W1's logit, which the
    kernel takes from round 1's list of tokens scoring at least 1/64 of the
    best.  Planted above the pivot:
    - W2, score (s1/64)(1 + 2e-5), whose word has ~w in [2^k, 2^k (1 + 2^-11)]
      with k in 21..22 (1 - u about 5e-4 to 1e-3, where the screen's bound on
      log2 E is within 1e-3 of log2 E): the proposal, inside the nucleus;
    - a decoy D, score (s1/64)(1 + 1e-5), far from the screen's edge, above
      W2 and inside the nucleus: the proposal, and the accepted token, if
      the list lost W2;
    - the max token M (weight 1, the row's largest E, score s1/70) and ~20
      filler tokens between W1 and W2, all scoring below s1/64;
    every other token below W1 with a score below s1.  p sits halfway
    between the masses strictly above W2 and above W1, so W2 is accepted in
    round 2 and W1 rejected in round 1.
    Returns (logits [B, V] f32, p [B] f32, seeds [B] u64, W1 [B], W2 [B], D [B])."""
    rng = np.random.default_rng(base_seed ^ 0x3C3C)
    logits = np.empty((B, V), np.float32)
    P = np.empty(B, np.float32)
    seeds = np.empty(B, np.uint64)
    w1s = np.empty(B, np.int64)
    w2s = np.empty(B, np.int64)
    ds = np.empty(B, np.int64)
    idx = np.arange(V)
    for b in range(B):
        for t in range(4096):
            sd = base_seed + 4096 * b + t
            words = orc.noise_words(sd, step, b, V)
            E = -np.log((words.astype(np.float64) + 0.5) * 2.0 ** -32)
            i1 = int(np.argmin(E))
            if E[i1] > 4e-6:
                continue
            n = (~words).astype(np.uint64)
            k = np.floor(np.log2(np.maximum(n, 1).astype(np.float64))).astype(np.int64)
            frac = n.astype(np.float64) / np.exp2(k) - 1.0
            ok = (k >= 21) & (k <= 22) & (frac <= 2.0 ** -11) & (idx >= V // 4) & ((idx % 2048) >= 512)
            ok[i1] = False
            if ok.any():
                break
        else:
            raise RuntimeError(f"row {b}: no key in 4096 gives the planted tokens")
        i2 = int(rng.choice(idx[ok]))
        iM = int(np.argmax(np.where(idx == i2, -np.inf, E)))
        dcand = idx[(E > 0.5) & (E < 2.0) & (idx != i1) & (idx != i2) & (idx != iM)]
        iD = int(rng.choice(dcand))
        s1 = 70.0 / E[iM]
        e = np.empty(V)
        e1 = s1 * E[i1]
        # Every other token: below W1 in weight and in score.
        e[:] = e1 * 0.9 * rng.uniform(0.01, 1.0, V)
        e[i1] = e1
        e[iM] = 1.0
        e[i2] = s1 / 64.0 * (1.0 + 2e-5) * E[i2]
        e[iD] = s1 / 64.0 * (1.0 + 1e-5) * E[iD]
        # Fillers between W1 and W2, scoring below s1/64 (their E is large).
        fc = idx[(E > 0.05) & (idx != i1) & (idx != i2) & (idx != iM) & (idx != iD)]
        fill = rng.choice(fc, 20, replace=False)
        lo, hi = e1 * 1.2, e[i2] * 0.8
        e[fill] = rng.uniform(lo, hi, 20)
        assert np.all(e[fill] / E[fill] < s1 / 64.0 * (1.0 - 1e-4))
        x = np.log(e).astype(np.float32)
        logits[b] = x
        ef = np.exp(x.astype(np.float64))
        S = ef.sum()
        a2 = ef[ef > ef[i2]].sum()
        a1 = ef[ef > ef[i1]].sum()
        P[b] = np.float32((a1 + a2) / (2.0 * S))
        seeds[b] = sd
        w1s[b] = i1
        w2s[b] = i2
        ds[b] = iD
    return logits, P, seeds, w1s, w2s, ds
