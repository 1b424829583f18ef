"""ctypes wrapper of the float64 CPU oracle (``nucleus_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

Parity unpinned by the pages: the Philox4x32-10 word stream (the pages fix no
key/counter layout or known-answer vectors); it is pinned in the tests against
rocRAND's independent Philox4x32-10 engine instead.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nucleus_oracle.c")
LIB_PATH = os.path.join(_HERE, "libnucleus_oracle.so")

F32, BF16 = 0, 1

# Mirrors of the C structs (natural alignment, same field order).
ROW_DTYPE = np.dtype(
    [
        ("status", np.int32), ("token", np.int32), ("keep_count", np.int32),
        ("n_survivors", np.int32), ("greedy", np.int32), ("topp_active", np.int32),
        ("min_kept_logit", np.float64), ("s_keep", np.float64), ("s_surv", np.float64),
        ("a_star", np.float64), ("m_star", np.float64), ("race_s1", np.float64),
        ("race_s2", np.float64), ("race_margin", np.float64), ("minp_nearest", np.float64),
    ],
    align=True,
)
REJ_DTYPE = np.dtype(
    [
        ("status", np.int32), ("token", np.int32), ("rounds", np.int32), ("greedy", np.int32),
        ("band", np.float64), ("race_margin", np.float64),
    ],
    align=True,
)
SPEC_DTYPE = np.dtype(
    [
        ("status", np.int32), ("token", np.int32), ("accepted", np.int32), ("greedy", np.int32),
        ("p_draft", np.float64), ("q_draft", np.float64), ("u", np.float64), ("s1", np.float64),
        ("s1_low", np.float64), ("threat", np.float64),
    ],
    align=True,
)
CUT_DTYPE = np.dtype(
    [
        ("status", np.int32), ("token", np.int32), ("keep_count", np.int32), ("pad", np.int32),
        ("a_cut", np.float64), ("m_cut", np.float64), ("s_keep", np.float64), ("race_s1", np.float64),
    ],
    align=True,
)


def build(force: bool = True, src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (plain C11, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", out, src, "-lm"]
        subprocess.run(cmd, check=True)
    return out


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(logits: np.ndarray) -> int:
    if logits.dtype == np.float32:
        return F32
    if logits.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError("oracle logits must be float32 or uint16 (bf16 bits)")


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str = LIB_PATH):
        L = ctypes.CDLL(path)
        vp, i64, u64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32
        L.oracle_sample.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, u64, u64, i64, i64, vp, vp]
        L.oracle_sample.restype = ctypes.c_int
        L.oracle_sample_ex.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, u64, vp, u64, i64, i64, vp,
                                       vp, vp]
        L.oracle_sample_ex.restype = ctypes.c_int
        L.oracle_sample_rejection.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, u64, vp, u64, i32, i64,
                                              i64, vp]
        L.oracle_sample_rejection.restype = ctypes.c_int
        L.oracle_spec_verify.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp, u64, vp, u64,
                                         ctypes.c_double, i64, i64, vp]
        L.oracle_spec_verify.restype = ctypes.c_int
        L.oracle_preprocess.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp]
        L.oracle_preprocess.restype = ctypes.c_int
        L.oracle_eval_cut.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_float, ctypes.c_float, i32,
                                      ctypes.c_float, u64, u64, ctypes.c_double, vp, vp]
        L.oracle_eval_cut.restype = ctypes.c_int
        L.oracle_race_score.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_float, u64, u64, i64]
        L.oracle_race_score.restype = ctypes.c_double
        L.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        L.oracle_philox4x32_10.restype = None
        L.oracle_noise_word.argtypes = [u64, u64, i64, i64]
        L.oracle_noise_word.restype = ctypes.c_uint32
        L.oracle_noise_words.argtypes = [u64, u64, i64, i64, vp]
        L.oracle_noise_words.restype = None
        L.oracle_exp1.argtypes = [ctypes.c_uint32]
        L.oracle_exp1.restype = ctypes.c_double
        L.oracle_topp_levels.argtypes = [vp, vp, i64, ctypes.c_double, vp, vp, vp]
        L.oracle_topp_levels.restype = i64
        self.L = L

    def sample(self, logits, temperature, top_p, top_k=None, min_p=None, seed=0, step=0,
               rows=None, want_probs=False, threads=1, seeds=None, want_logprobs=False):
        """Run the oracle on a [B, V] batch.

        ``logits`` is float32 or uint16 (bf16 bit patterns).  ``rows``
        (optional iterable of row indices) limits the work to those rows; the
        other entries of the result stay zero.  ``seeds`` (optional [B]
        uint64) gives each row its own race key.  Returns (rows, probs): a
        structured array of ROW_DTYPE of length B, and float64 probabilities
        ([B, V], or [len(rows), V] in the order of ``rows``) or None; with
        ``want_logprobs``, (rows, probs, logprobs), the log-probabilities laid
        out like the probabilities.
        """
        logits = np.ascontiguousarray(logits)
        B, V = logits.shape
        dt = _dtype_code(logits)
        T = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
        P = np.ascontiguousarray(top_p, dtype=np.float32).reshape(B)
        K = None if top_k is None else np.ascontiguousarray(top_k, dtype=np.int32).reshape(B)
        MP = None if min_p is None else np.ascontiguousarray(min_p, dtype=np.float32).reshape(B)
        S = None if seeds is None else np.ascontiguousarray(seeds, dtype=np.uint64).reshape(B)
        out = np.zeros(B, dtype=ROW_DTYPE)
        if rows is None:
            spans = [(b, b + 1) for b in range(B)] if threads > 1 else [(0, B)]
        else:
            spans = [(int(b), int(b) + 1) for b in rows]
        # probs[j] belongs to spans[j][0] .. (one buffer row per span row)
        nrows = sum(s1 - s0 for s0, s1 in spans)
        probs = np.zeros((nrows, V), dtype=np.float64) if want_probs else None
        logprobs = np.zeros((nrows, V), dtype=np.float64) if want_logprobs else None
        starts = np.cumsum([0] + [s1 - s0 for s0, s1 in spans])
        L = self.L

        def run(j):
            s0, s1 = spans[j]
            pp = None if probs is None else probs[starts[j]:starts[j + 1]]
            lp = None if logprobs is None else logprobs[starts[j]:starts[j + 1]]
            rc = L.oracle_sample_ex(_ptr(logits), dt, B, V, V, _ptr(T), _ptr(P), _ptr(K), _ptr(MP),
                                    ctypes.c_uint64(seed), _ptr(S), ctypes.c_uint64(step), s0, s1, _ptr(out),
                                    None if pp is None else pp.ctypes.data, None if lp is None else lp.ctypes.data)
            if rc != 0:
                raise ValueError("oracle_sample rejected its arguments")

        if threads > 1 and len(spans) > 1:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, range(len(spans))))
        else:
            for j in range(len(spans)):
                run(j)
        if want_logprobs:
            return out, probs, logprobs
        return out, probs

    def sample_rejection(self, logits, temperature, top_p, min_p=None, seed=0, step=0, seeds=None,
                         max_rounds=64, threads=1):
        """The rejection sampler (oracle_sample_rejection) on a [B, V] batch.
        Returns a structured array of REJ_DTYPE of length B."""
        logits = np.ascontiguousarray(logits)
        B, V = logits.shape
        dt = _dtype_code(logits)
        T = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
        P = np.ascontiguousarray(top_p, dtype=np.float32).reshape(B)
        MP = None if min_p is None else np.ascontiguousarray(min_p, dtype=np.float32).reshape(B)
        S = None if seeds is None else np.ascontiguousarray(seeds, dtype=np.uint64).reshape(B)
        out = np.zeros(B, dtype=REJ_DTYPE)
        L = self.L

        def run(span):
            rc = L.oracle_sample_rejection(_ptr(logits), dt, B, V, V, _ptr(T), _ptr(P), _ptr(MP),
                                           ctypes.c_uint64(seed), _ptr(S), ctypes.c_uint64(step), int(max_rounds),
                                           span[0], span[1], _ptr(out))
            if rc != 0:
                raise ValueError("oracle_sample_rejection rejected its arguments")

        n = max(1, min(threads, B))
        edges = np.linspace(0, B, n + 1).astype(np.int64)
        spans = [(int(edges[j]), int(edges[j + 1])) for j in range(n) if edges[j + 1] > edges[j]]
        if len(spans) > 1:
            with ThreadPoolExecutor(len(spans)) as ex:
                list(ex.map(run, spans))
        else:
            for sp in spans:
                run(sp)
        return out

    def spec_verify(self, logits, temperature, top_p, top_k, min_p, draft_probs, draft_token, seed=0, step=0,
                    seeds=None, rel_tol=2e-5, threads=1):
        """Speculative acceptance (oracle_spec_verify) on a [B, V] batch:
        ``draft_probs`` [B, V] float32, ``draft_token`` [B].  Returns a
        structured array of SPEC_DTYPE of length B."""
        logits = np.ascontiguousarray(logits)
        B, V = logits.shape
        dt = _dtype_code(logits)
        T = np.ascontiguousarray(temperature, dtype=np.float32).reshape(B)
        P = np.ascontiguousarray(top_p, dtype=np.float32).reshape(B)
        K = None if top_k is None else np.ascontiguousarray(top_k, dtype=np.int32).reshape(B)
        MP = None if min_p is None else np.ascontiguousarray(min_p, dtype=np.float32).reshape(B)
        Q = np.ascontiguousarray(draft_probs, dtype=np.float32).reshape(B, V)
        D = np.ascontiguousarray(draft_token, dtype=np.int32).reshape(B)
        S = None if seeds is None else np.ascontiguousarray(seeds, dtype=np.uint64).reshape(B)
        out = np.zeros(B, dtype=SPEC_DTYPE)
        L = self.L

        def run(span):
            rc = L.oracle_spec_verify(_ptr(logits), dt, B, V, V, _ptr(T), _ptr(P), _ptr(K), _ptr(MP), _ptr(Q), _ptr(D),
                                      ctypes.c_uint64(seed), _ptr(S), ctypes.c_uint64(step), float(rel_tol),
                                      span[0], span[1], _ptr(out))
            if rc != 0:
                raise ValueError("oracle_spec_verify rejected its arguments")

        n = max(1, min(threads, B))
        edges = np.linspace(0, B, n + 1).astype(np.int64)
        spans = [(int(edges[j]), int(edges[j + 1])) for j in range(n) if edges[j + 1] > edges[j]]
        if len(spans) > 1:
            with ThreadPoolExecutor(len(spans)) as ex:
                list(ex.map(run, spans))
        else:
            for sp in spans:
                run(sp)
        return out

    def preprocess(self, logits, hist=None, repetition=None, frequency=None, presence=None, allowed=None):
        """The pre-chain (oracle_preprocess): penalised, masked fp32 logits
        [B, V].  ``hist`` [B, H] int32 (-1 padded), penalties [B] float32,
        ``allowed`` [B, ceil(V/32)] uint32 bit masks."""
        logits = np.ascontiguousarray(logits)
        B, V = logits.shape
        Hs = None if hist is None else np.ascontiguousarray(hist, dtype=np.int32).reshape(B, -1)
        H = 0 if Hs is None else Hs.shape[1]

        def vec(a):
            return None if a is None else np.ascontiguousarray(a, dtype=np.float32).reshape(B)

        R, F, Pp = vec(repetition), vec(frequency), vec(presence)
        M = None if allowed is None else np.ascontiguousarray(allowed, dtype=np.uint32).reshape(B, (V + 31) // 32)
        out = np.empty((B, V), np.float32)
        rc = self.L.oracle_preprocess(_ptr(logits), _dtype_code(logits), B, V, V, _ptr(Hs), H, _ptr(R), _ptr(F),
                                      _ptr(Pp), _ptr(M), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_preprocess rejected its arguments")
        return out

    def eval_cut(self, logits_row, row, temperature, top_p, top_k, min_p, seed, step, cut, want_probs=False):
        """Judge a keep threshold chosen elsewhere on one row (see oracle_eval_cut)."""
        logits_row = np.ascontiguousarray(logits_row)
        V = logits_row.shape[-1]
        out = np.zeros(1, dtype=CUT_DTYPE)
        probs = np.zeros(V, dtype=np.float64) if want_probs else None
        rc = self.L.oracle_eval_cut(_ptr(logits_row), _dtype_code(logits_row), V, 0, int(row),
                                    float(temperature), float(top_p), int(top_k), float(min_p),
                                    ctypes.c_uint64(seed), ctypes.c_uint64(step), float(cut), _ptr(out),
                                    _ptr(probs))
        if rc != 0:
            raise ValueError("oracle_eval_cut rejected its arguments")
        return out[0], probs

    def race_score(self, logits_row, row, temperature, seed, step, token):
        logits_row = np.ascontiguousarray(logits_row)
        return self.L.oracle_race_score(_ptr(logits_row), _dtype_code(logits_row), logits_row.shape[-1], 0,
                                        int(row), float(temperature), ctypes.c_uint64(seed),
                                        ctypes.c_uint64(step), int(token))

    def philox4x32_10(self, counter, key):
        c = np.ascontiguousarray(counter, dtype=np.uint32)
        k = np.ascontiguousarray(key, dtype=np.uint32)
        o = np.zeros(4, dtype=np.uint32)
        self.L.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
        return o

    def noise_word(self, seed, step, row, token):
        return int(self.L.oracle_noise_word(ctypes.c_uint64(seed), ctypes.c_uint64(step), int(row), int(token)))

    def noise_words(self, seed, step, row, n):
        """Words of tokens 0 .. n-1 of one row (oracle_noise_words)."""
        out = np.zeros(int(n), dtype=np.uint32)
        self.L.oracle_noise_words(ctypes.c_uint64(seed), ctypes.c_uint64(step), int(row), int(n), _ptr(out))
        return out

    def exp1(self, word):
        return float(self.L.oracle_exp1(int(word)))

    def topp_levels(self, order, mass, p):
        """Probability-level top-p rule: returns (keep bool array, a_star, m_star)."""
        order = np.ascontiguousarray(order, dtype=np.float64)
        mass = np.ascontiguousarray(mass, dtype=np.float64)
        n = order.shape[0]
        keep = np.zeros(n, dtype=np.uint8)
        a = np.zeros(1)
        m = np.zeros(1)
        self.L.oracle_topp_levels(_ptr(order), _ptr(mass), n, float(p), _ptr(keep), _ptr(a), _ptr(m))
        return keep.astype(bool), float(a[0]), float(m[0])


_default = None


def stale() -> bool:
    """True when the built library is missing or older than its source."""
    return not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)


def default() -> Oracle:
    """The oracle built from this directory's source (rebuilt when stale)."""
    global _default
    if _default is None:
        if stale():
            build(force=True)
        _default = Oracle(LIB_PATH)
    return _default


def sample(*a, **k):
    return default().sample(*a, **k)


def sample_rejection(*a, **k):
    return default().sample_rejection(*a, **k)


def spec_verify(*a, **k):
    return default().spec_verify(*a, **k)


def preprocess(*a, **k):
    return default().preprocess(*a, **k)


def eval_cut(*a, **k):
    return default().eval_cut(*a, **k)


def race_score(*a, **k):
    return default().race_score(*a, **k)


def philox4x32_10(*a, **k):
    return default().philox4x32_10(*a, **k)


def noise_word(*a, **k):
    return default().noise_word(*a, **k)


def noise_words(*a, **k):
    return default().noise_words(*a, **k)


def exp1(*a, **k):
    return default().exp1(*a, **k)


def topp_levels(*a, **k):
    return default().topp_levels(*a, **k)
