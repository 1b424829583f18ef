"""Seeded synthetic inputs for batched nucleus sampling.

This module only draws inputs: logits and per-row parameters.  It holds none
of the sampling arithmetic and is shared by the tests, the smoke check and the
benchmark; both the GPU library and the oracle receive exactly these arrays.

Every row is generated from its own NumPy PCG64 stream seeded by
(1000 + workload number, row), so any subset of rows can be regenerated
without generating the whole batch.  The Philox key of workload n is
0x5EED0000 + n.

Workloads (logit shapes and distributions stand in for real LM-head output;
no model, dataset or trained weights are involved):

1. ``small``   B = 8 + 7, V = 1024 fp32.  Eight rows of Normal(0, 2) logits,
   T cycling {0, 0.7, 1.0, 1.5}, p ~ U[0.05, 1.0] with row 3 at exactly 1.0,
   no top-k, no min-p.  Then the pages' worked-example rows, padded with -inf
   to V: [4, 3, 2.2, 1.6, 1, -2] at p = 0.5 and 0.9; [3, 2.5, 2, 1, 0.5, 0]
   at p = 0.9 with T = 0.7, 1.0, 1.5; a 100-token peaked row (8, 3, 2, 1,
   then zeros) and a 100-token row evenly spaced from 1 to 0, both at p = 0.9.
2. ``ties``    B = 64, V = 32000 fp32.  Even rows Normal(0, 1) with three
   random tokens raised by +8; odd rows drawn from the integers {-2..2} so
   ties straddle the cut.  T ~ U[0.5, 2], p ~ U[0.3, 1].
3. ``zipf``    B = 256, V = 128256 fp32.  z_i = -1.1 ln(rank_i) + Normal(0, 0.5)
   with ranks a random permutation of 1..V; T ~ U[0.3, 1.5], p ~ U[0.8, 0.99].
4. ``chain``   B = 256, V = 128256 bf16 (round to nearest even) of Normal(0, 3)
   with 5 % of tokens set to -inf; T = 0 on rows b % 8 == 0, else 0.7 on odd
   and 1.0 on even rows; min_p = 0.05; top_k = 50 on even rows, else 0; p = 0.9.
5. ``flat``    B = 1024, V = 152064 fp32.  linspace(1, 0, V) over a random
   permutation plus Normal(0, 0.01); p = 1.0 on 10 % of rows, 1e-4 on 10 %,
   else U[0.5, 1.0); T ~ U[0.8, 1.2].
"""
from __future__ import annotations

import numpy as np

NAMES = {1: "small", 2: "ties", 3: "zipf", 4: "chain", 5: "flat"}
SHAPES = {1: (15, 1024), 2: (64, 32000), 3: (256, 128256), 4: (256, 128256), 5: (1024, 152064)}
DTYPES = {1: "f32", 2: "f32", 3: "f32", 4: "bf16", 5: "f32"}


def philox_seed(n: int) -> int:
    return 0x5EED0000 + n


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    -inf stays -inf; the inputs here hold no NaN."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32)


def _fixed_rows_small(V: int):
    """The pages' worked examples, as (logits, T, p) rows padded with -inf."""
    six = [4.0, 3.0, 2.2, 1.6, 1.0, -2.0]
    tab = [3.0, 2.5, 2.0, 1.0, 0.5, 0.0]
    peaked = [8.0, 3.0, 2.0, 1.0] + [0.0] * 96
    sloped = list(np.linspace(1.0, 0.0, 100))
    spec = [(six, 1.0, 0.5), (six, 1.0, 0.9), (tab, 0.7, 0.9), (tab, 1.0, 0.9), (tab, 1.5, 0.9),
            (peaked, 1.0, 0.9), (sloped, 1.0, 0.9)]
    out = []
    for vals, T, p in spec:
        row = np.full(V, -np.inf, dtype=np.float32)
        row[: len(vals)] = np.asarray(vals, dtype=np.float32)
        out.append((row, T, p))
    return out


def _row(n: int, b: int, V: int):
    """(logits_row, T, p, k, min_p) of row b of workload n."""
    rng = np.random.default_rng([1000 + n, b])
    if n == 1:
        if b < 8:
            T = (0.0, 0.7, 1.0, 1.5)[b % 4]
            p = 1.0 if b == 3 else rng.uniform(0.05, 1.0)
            return rng.normal(0.0, 2.0, V).astype(np.float32), T, p, 0, 0.0
        row, T, p = _fixed_rows_small(V)[b - 8]
        return row, T, p, 0, 0.0
    if n == 2:
        T = rng.uniform(0.5, 2.0)
        p = rng.uniform(0.3, 1.0)
        if b % 2 == 0:
            z = rng.normal(0.0, 1.0, V)
            z[rng.choice(V, 3, replace=False)] += 8.0
        else:
            z = rng.integers(-2, 3, V).astype(np.float64)
        return z.astype(np.float32), T, p, 0, 0.0
    if n == 3:
        T = rng.uniform(0.3, 1.5)
        p = rng.uniform(0.8, 0.99)
        rank = rng.permutation(V) + 1
        z = -1.1 * np.log(rank.astype(np.float64)) + rng.normal(0.0, 0.5, V)
        return z.astype(np.float32), T, p, 0, 0.0
    if n == 4:
        T = 0.0 if b % 8 == 0 else (0.7 if b % 2 == 1 else 1.0)
        k = 50 if b % 2 == 0 else 0
        z = rng.normal(0.0, 3.0, V).astype(np.float32)
        z[rng.random(V) < 0.05] = -np.inf
        return z, T, 0.9, k, 0.05
    if n == 5:
        u = rng.random()
        p = 1.0 if u < 0.1 else (1e-4 if u < 0.2 else rng.uniform(0.5, 1.0))
        T = rng.uniform(0.8, 1.2)
        z = np.linspace(1.0, 0.0, V)[rng.permutation(V)] + rng.normal(0.0, 0.01, V)
        return z.astype(np.float32), T, p, 0, 0.0
    raise ValueError(f"unknown workload {n}")


def make(n: int, rows=None):
    """Inputs of workload n (optionally only the given rows, in that order).

    Returns a dict: logits (float32 [B, V], or uint16 bf16 bits for the bf16
    workload), dtype ('f32'|'bf16'), temperature, top_p (float32 [B]), top_k
    (int32 [B]), min_p (float32 [B]), seed (Philox key), rows (the row ids,
    which are also the rows' Philox counter values).
    """
    B, V = SHAPES[n]
    ids = np.arange(B) if rows is None else np.asarray(list(rows), dtype=np.int64)
    L = np.empty((len(ids), V), dtype=np.float32)
    T = np.empty(len(ids), np.float32)
    P = np.empty(len(ids), np.float32)
    K = np.empty(len(ids), np.int32)
    MP = np.empty(len(ids), np.float32)
    for j, b in enumerate(ids):
        L[j], T[j], P[j], K[j], MP[j] = _row(n, int(b), V)
    logits = f32_to_bf16_bits(L) if DTYPES[n] == "bf16" else L
    return dict(logits=logits, dtype=DTYPES[n], temperature=T, top_p=P, top_k=K, min_p=MP,
                seed=philox_seed(n), rows=ids, name=NAMES[n], B=len(ids), V=V)


def make_draft(w: dict, noise: float = 0.7, keep_top: int = 64, seed: int = 0):
    """A draft model's sampling distribution and its sampled tokens for the
    rows of workload dict ``w`` (for speculative-decoding verification):
    q = softmax((x + N(0, noise)) / Td) per row, Td = T (0.7 on greedy rows),
    -inf logits get q = 0; odd rows are truncated to the draft's own top
    ``keep_top`` tokens and renormalised (a draft that applies truncation).
    The draft token of each row is drawn from q.  Returns (q float32 [B, V],
    d int32 [B]).  Each row has its own PCG64 stream (seed, 77, row)."""
    x = w["logits"]
    x = bf16_bits_to_f32(x) if w["dtype"] == "bf16" else x
    B, V = x.shape
    q = np.zeros((B, V), np.float32)
    d = np.zeros(B, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, 77, b])
        T = float(w["temperature"][b])
        Td = T if T > 0 and np.isfinite(T) else 0.7
        row = x[b].astype(np.float64)
        fin = np.isfinite(row)
        z = np.where(fin, row + rng.normal(0.0, noise, V), -np.inf) / Td
        if not fin.any():
            z = rng.normal(0.0, 1.0, V)
        z = z - z[np.isfinite(z)].max()
        e = np.where(np.isfinite(z), np.exp(z), 0.0)
        if b % 2 == 1 and keep_top < V:
            cut = np.partition(e, V - keep_top)[V - keep_top]
            e = np.where(e >= cut, e, 0.0)
        qq = (e / e.sum()).astype(np.float32)
        q[b] = qq
        c = np.cumsum(qq.astype(np.float64))
        d[b] = min(int(np.searchsorted(c, rng.random() * c[-1], side="right")), V - 1)
        while d[b] > 0 and qq[d[b]] == 0.0:  # land on a token the draft can propose
            d[b] -= 1
    return q, d


def make_prechain(w: dict, hist_len: int = 256, seed: int = 0):
    """Synthetic pre-chain inputs for the rows of workload dict ``w``: a
    generated-token history per row (tokens drawn from the row's highest
    logits and at random, duplicates included, -1 padded to ``hist_len``),
    repetition / frequency / presence penalties (a quarter of the rows
    without any), and a grammar bit mask forbidding about a fifth of the
    vocabulary at random plus, on every third row, the row's top token (all
    tokens allowed on every fifth row).  Returns a dict of NumPy arrays:
    history [B, H] int32, repetition / frequency / presence [B] float32,
    allowed [B, ceil(V/32)] uint32."""
    x = w["logits"]
    x = bf16_bits_to_f32(x) if w["dtype"] == "bf16" else x
    B, V = x.shape
    W = (V + 31) // 32
    hist = np.full((B, hist_len), -1, np.int32)
    rep = np.ones(B, np.float32)
    fr = np.zeros(B, np.float32)
    pr = np.zeros(B, np.float32)
    allowed = np.full((B, W), 0xFFFFFFFF, np.uint32)
    for b in range(B):
        rng = np.random.default_rng([seed, 91, b])
        n = int(rng.integers(0, hist_len + 1))
        top = np.argsort(-np.nan_to_num(x[b].astype(np.float64), nan=-np.inf))[: max(1, min(V, 32))]
        picks = np.where(rng.random(n) < 0.6, rng.choice(top, n), rng.integers(0, V, n))
        hist[b, :n] = picks
        if b % 4 != 3:
            rep[b] = np.float32(rng.choice([1.0, 1.1, 1.3, 2.0]))
            fr[b] = np.float32(rng.uniform(0, 0.5))
            pr[b] = np.float32(rng.uniform(0, 0.5))
        if b % 5 != 4:
            bits = rng.random(W * 32) >= 0.2
            if b % 3 == 0:
                bits[int(top[0])] = False
            bits[V:] = True
            words = np.packbits(bits.reshape(W, 32)[:, ::-1], axis=1, bitorder="big").view(">u4").astype(np.uint32)
            allowed[b] = words.reshape(W)
    return dict(history=hist, repetition=rep, frequency=fr, presence=pr, allowed=allowed)
