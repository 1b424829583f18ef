"""Row-by-row comparison of sampler outputs with the oracle.

TEST INFRASTRUCTURE ONLY: used by the GPU parity tests and the smoke check.

Rules, per row b (p = top_p[b]):

* row error (oracle status 1): token -1, keep count 0, min kept logit NaN,
  probabilities all zero.
* greedy (T <= 0): token, keep count 1 and one-hot probabilities exactly.
* otherwise, unless exempt: keep count and smallest kept logit exactly (so the
  keep mask is exactly the oracle's), token exactly, probabilities within
  |gpu - oracle| <= 1e-6 + 1e-5 * oracle.
* mass-band exemption: the oracle's mass above the last kept level (A*) or
  above the first dropped one (M*) lies within 1e-5 of p.  The row is then
  judged by the admissible-set rule: the GPU's cut level L must satisfy
  A(L) < p + 1e-5 and M(L) >= p - 1e-5 under the oracle's masses, and the
  GPU's count, token and probabilities must equal the oracle's evaluation of
  that same cut.  Exact agreement on exempt rows is counted separately.
* race exemption: the oracle's race margin (s1 - s2)/s1 is below 1e-6.  The
  GPU's token must then be kept and score at least s1 (1 - 1e-6) under the
  oracle.
* min-p boundary: a token whose p_i/(min_p p_max) lies within 1e-9 of 1 can
  fall either way; such rows are counted and only checked for validity.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import default as _default_oracle

MASS_BAND = 1e-5
RACE_BAND = 1e-6
MINP_BAND = 1e-9


@dataclass
class Report:
    rows: int = 0
    exact: int = 0
    errors_ok: int = 0
    greedy: int = 0
    exempt_mass: int = 0
    exempt_mass_exact: int = 0
    exempt_race: int = 0
    exempt_minp: int = 0
    near_1e6: int = 0
    near_1e7: int = 0
    max_prob_ratio: float = 0.0
    max_logprob_ratio: float = 0.0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        return (f"rows={self.rows} exact={self.exact} greedy={self.greedy} row_errors={self.errors_ok} "
                f"exempt_mass={self.exempt_mass} (exact {self.exempt_mass_exact}) exempt_race={self.exempt_race} "
                f"exempt_minp={self.exempt_minp} band1e-6={self.near_1e6} band1e-7={self.near_1e7} "
                f"max|dp|/(1e-6+1e-5p)={self.max_prob_ratio:.3g} "
                f"max|dlp|/(1e-6+1e-6|lp|)={self.max_logprob_ratio:.3g} failures={len(self.failures)}")


def _prob_ratio(g, o):
    return float(np.max(np.abs(g - o) / (1e-6 + 1e-5 * o))) if g.size else 0.0


# Log-probabilities: the GPU forms (x - m)/T to about 2^-48 relative and
# ln S_keep from the bin model's sums (about 1e-7 relative in S_keep, 1e-7
# absolute in its log), then rounds to float32 (2^-24 |lp| per operation):
# |gpu - oracle| <= 1e-6 + 1e-6 |lp| holds with margin.  Both sides must put
# -inf on exactly the same tokens.
def _logprob_ratio(g, o):
    fin = np.isfinite(o)
    if not np.array_equal(fin, np.isfinite(g)) or not np.array_equal(np.isneginf(o), np.isneginf(g)):
        return float("inf")
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(g[fin] - o[fin]) / (1e-6 + 1e-6 * np.abs(o[fin]))))


def compare(logits, temperature, top_p, top_k, min_p, seed, step, gpu_token, gpu_count, gpu_min_kept,
            oracle_rows, gpu_probs=None, oracle_probs=None, prob_rows=None, batch_rows=None, O=None,
            max_failures=20, seeds=None, gpu_logprobs=None, oracle_logprobs=None) -> Report:
    """Compare GPU outputs with oracle results.

    logits: host [B, V] (float32 or uint16 bf16 bits) as given to both sides.
    gpu_*: host arrays [B]; oracle_rows: ROW_DTYPE [B].
    gpu_probs / oracle_probs, gpu_logprobs / oracle_logprobs: optional [R, V]
    for the rows listed in prob_rows.
    batch_rows: the Philox row index of each row (defaults to 0..B-1).
    seeds: optional per-row race keys (row b then uses seeds[b], not seed).
    """
    O = O or _default_oracle()
    B = logits.shape[0]
    T = np.asarray(temperature, np.float32)
    P = np.asarray(top_p, np.float32)
    K = np.zeros(B, np.int32) if top_k is None else np.asarray(top_k, np.int32)
    MP = np.zeros(B, np.float32) if min_p is None else np.asarray(min_p, np.float32)
    rid = np.arange(B) if batch_rows is None else np.asarray(batch_rows)
    prob_index = {} if prob_rows is None else {int(b): j for j, b in enumerate(prob_rows)}
    rep = Report()

    def fail(b, why):
        if len(rep.failures) < max_failures:
            rep.failures.append((int(b), why))
        else:
            rep.failures.append((int(b), "..."))

    for b in range(B):
        rep.rows += 1
        o = oracle_rows[b]
        gt, gc, gm = int(gpu_token[b]), int(gpu_count[b]), float(gpu_min_kept[b]) if gpu_min_kept is not None else None
        j = prob_index.get(b)
        gp = gpu_probs[j] if (j is not None and gpu_probs is not None) else None
        op = oracle_probs[j] if (j is not None and oracle_probs is not None) else None
        gl = gpu_logprobs[j] if (j is not None and gpu_logprobs is not None) else None
        ol = oracle_logprobs[j] if (j is not None and oracle_logprobs is not None) else None
        sb = int(seeds[b]) if seeds is not None else seed
        if o["status"] == 1:
            good = gt == -1 and gc == 0 and (gm is None or math.isnan(gm)) and (gp is None or not gp.any())
            good &= gl is None or bool(np.all(np.isnan(gl)))
            if good:
                rep.errors_ok += 1
            else:
                fail(b, f"row error expected, got token={gt} count={gc} min_kept={gm}")
            continue
        if o["greedy"]:
            rep.greedy += 1
            good = gt == o["token"] and gc == 1 and (gm is None or gm == o["min_kept_logit"])
            if gp is not None:
                good &= gp[gt] == 1.0 and np.count_nonzero(gp) == 1
            if gl is not None:
                good &= gl[gt] == 0.0 and int(np.isneginf(gl).sum()) == len(gl) - 1
            if good:
                rep.exact += 1
            else:
                fail(b, f"greedy: token {gt} vs {o['token']}, count {gc}, min_kept {gm} vs {o['min_kept_logit']}")
            continue
        p = float(P[b])
        a_s, m_s = float(o["a_star"]), float(o["m_star"])
        if o["topp_active"]:
            d = min(abs(a_s - p), abs(m_s - p))
            rep.near_1e6 += d <= 1e-6
            rep.near_1e7 += d <= 1e-7
        exempt_mass = bool(o["topp_active"]) and (abs(a_s - p) <= MASS_BAND or abs(m_s - p) <= MASS_BAND)
        exempt_minp = float(o["minp_nearest"]) <= MINP_BAND
        same_set = gc == o["keep_count"] and gm is not None and gm == o["min_kept_logit"]
        if exempt_minp:
            rep.exempt_minp += 1
            if not (0 <= gt < logits.shape[1] and gc >= 1):
                fail(b, f"min-p boundary row: invalid token {gt} / count {gc}")
            continue
        if exempt_mass:
            rep.exempt_mass += 1
            if gm is None:
                fail(b, "mass-band row needs the GPU's min kept logit")
                continue
            ev, eprobs = O.eval_cut(logits[b], rid[b], T[b], P[b], K[b], MP[b], sb, step, gm,
                                    want_probs=gp is not None or gl is not None)
            if not (ev["a_cut"] < p + MASS_BAND and ev["m_cut"] >= p - MASS_BAND):
                fail(b, f"inadmissible cut {gm}: A={ev['a_cut']:.9f} M={ev['m_cut']:.9f} p={p:.9f}")
                continue
            if gc != ev["keep_count"]:
                fail(b, f"count {gc} does not match the cut's {ev['keep_count']}")
                continue
            want_tok, s1 = int(ev["token"]), float(ev["race_s1"])
            ref_probs = eprobs
            # (the cut's distribution in the log domain; the workloads' kept
            # probabilities are far from underflow)
            ref_lp = None
            if eprobs is not None:
                with np.errstate(divide="ignore"):
                    ref_lp = np.where(eprobs > 0, np.log(np.where(eprobs > 0, eprobs, 1.0)), -np.inf)
            if same_set:
                rep.exempt_mass_exact += 1
        else:
            if not same_set:
                fail(b, f"keep set: count {gc} vs {o['keep_count']}, min_kept {gm} vs {o['min_kept_logit']}")
                continue
            want_tok, s1 = int(o["token"]), float(o["race_s1"])
            ref_probs = op
            ref_lp = ol
        if gt != want_tok:
            margin = float(o["race_margin"]) if not exempt_mass else None
            sg = O.race_score(logits[b], rid[b], T[b], sb, step, gt) if 0 <= gt < logits.shape[1] else -1.0
            kept_ok = 0 <= gt < logits.shape[1] and _kept(logits[b], gt, gm)
            if kept_ok and sg >= s1 * (1.0 - RACE_BAND):
                rep.exempt_race += 1
            else:
                fail(b, f"token {gt} vs {want_tok} (oracle score {sg:.9g} vs best {s1:.9g}, margin {margin})")
                continue
        elif not exempt_mass:
            rep.exact += 1
        if gp is not None and ref_probs is not None:
            r = _prob_ratio(gp.astype(np.float64), ref_probs)
            rep.max_prob_ratio = max(rep.max_prob_ratio, r)
            if r > 1.0:
                fail(b, f"probabilities off by {r:.3g} x tolerance")
        if gl is not None and ref_lp is not None:
            r = _logprob_ratio(gl.astype(np.float64), ref_lp)
            rep.max_logprob_ratio = max(rep.max_logprob_ratio, r)
            if r > 1.0:
                fail(b, f"log-probabilities off by {r:.3g} x tolerance (or -inf on different tokens)")
    return rep


def _kept(row, tok, min_kept):
    x = row[tok]
    if row.dtype == np.uint16:
        x = np.asarray([x], np.uint16).astype(np.uint32) << 16
        x = x.view(np.float32)[0]
    return bool(np.isfinite(x) and x >= min_kept)


@dataclass
class RejectionReport:
    rows: int = 0
    exact: int = 0
    errors_ok: int = 0
    greedy: int = 0
    exempt: int = 0
    exempt_exact: int = 0
    rounds_total: int = 0
    rounds_max: int = 0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        drawn = max(self.rows - self.errors_ok - self.greedy, 1)
        return (f"rows={self.rows} exact={self.exact} greedy={self.greedy} row_errors={self.errors_ok} "
                f"exempt={self.exempt} (exact {self.exempt_exact}) rounds mean "
                f"{self.rounds_total / drawn:.3f} max {self.rounds_max} failures={len(self.failures)}")


def compare_rejection(logits, temperature, top_p, min_p, seed, step, gpu_token, gpu_rounds, orows, seeds=None):
    """Rejection sampler outputs against oracle_sample_rejection's rows.

    * row error: token -1, rounds 0.  Greedy (T <= 0): token exactly, rounds 0.
    * otherwise, unless exempt: token and rounds exactly.
    * exempt: some round's acceptance test lies within 1e-5 of p (|A(t)/S - p|)
      or some round's race within 1e-6 relative of a tie.  The GPU's token must
      then be admissible under the oracle's masses: a min-p survivor whose
      level has survivor mass above it < p + 1e-5 (any survivor for p >= 1),
      and its rounds in [1, 64].
    """
    O = _default_oracle()
    B, V = logits.shape
    rep = RejectionReport()
    for b in range(B):
        rep.rows += 1
        o = orows[b]
        g, gr = int(gpu_token[b]), int(gpu_rounds[b])
        if o["status"] == 1:
            if g == -1 and gr == 0:
                rep.errors_ok += 1
            else:
                rep.failures.append((b, f"row error: gpu token {g} rounds {gr}"))
            continue
        if o["greedy"]:
            rep.greedy += 1
            if g != int(o["token"]) or gr != 0:
                rep.failures.append((b, f"greedy: gpu {g}/{gr} oracle {int(o['token'])}"))
            continue
        rep.rounds_total += max(gr, 0)
        rep.rounds_max = max(rep.rounds_max, gr)
        exempt = o["band"] <= MASS_BAND or o["race_margin"] <= RACE_BAND or o["status"] == 2
        if not exempt:
            if g == int(o["token"]) and gr == int(o["rounds"]):
                rep.exact += 1
            else:
                rep.failures.append((b, f"gpu {g}/{gr} rounds, oracle {int(o['token'])}/{int(o['rounds'])} "
                                        f"(band {o['band']:.3g}, margin {o['race_margin']:.3g})"))
            continue
        rep.exempt += 1
        if g == int(o["token"]) and gr == int(o["rounds"]):
            rep.exempt_exact += 1
            continue
        if not (0 <= g < V and 1 <= gr <= 64):
            rep.failures.append((b, f"exempt row: gpu token {g} rounds {gr} out of range"))
            continue
        row = logits[b]
        mp = 0.0 if min_p is None else float(min_p[b])
        s = int(seeds[b]) if seeds is not None else seed
        if row.dtype == np.float32:
            xt = float(row[g])
        else:  # bf16 bits, widened exactly
            xt = float((np.asarray([row[g]], np.uint32) << 16).view(np.float32)[0])
        ev, _ = O.eval_cut(row, b, float(temperature[b]), float(top_p[b]), 0, mp, s, step, xt)
        p = float(top_p[b])
        # The token's own level must survive min-p (its survivor mass is m_cut - a_cut).
        survives = ev["m_cut"] > ev["a_cut"] or (mp <= 0.0 and math.isfinite(xt))
        ok = ev["status"] == 0 and survives and (p >= 1.0 or ev["a_cut"] == 0.0 or ev["a_cut"] < p + MASS_BAND)
        if not ok:
            rep.failures.append((b, f"exempt row: gpu token {g} not admissible (a_cut {ev['a_cut']:.6g}, p {p})"))
    return rep


SPEC_REL_TOL = 2e-5  # relative uncertainty of the GPU's kept probabilities (p within 1e-5 p, plus fp32 rounding)


@dataclass
class SpecReport:
    rows: int = 0
    exact: int = 0
    accepted: int = 0
    errors_ok: int = 0
    exempt_cut: int = 0
    exempt_accept: int = 0
    exempt_race: int = 0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        return (f"rows={self.rows} exact={self.exact} accepted={self.accepted} row_errors={self.errors_ok} "
                f"exempt_cut={self.exempt_cut} exempt_accept={self.exempt_accept} exempt_race={self.exempt_race} "
                f"failures={len(self.failures)}")


def compare_spec(draft_probs, draft_token, gpu_token, gpu_accepted, gpu_keep_count, gpu_p_at_token, orows,
                 otarget, top_p):
    """Speculative verification outputs against oracle_spec_verify's rows.

    * row error (oracle status 1): token -1, not accepted.  Nothing to
      resample (status 2): token -1.
    * the GPU's target kept a different set than the oracle: allowed only
      for a row within the mass band of its cut (the oracle's A* or M* within
      MASS_BAND of p, the target's own exemption rule); the output must then
      be valid for the GPU's own p: the draft token if accepted, else a token
      with p > q.  A different set on any other row is a failure.
    * the acceptance test within SPEC_REL_TOL p(d) of its boundary: valid as
      above.  Otherwise acceptance exactly; an accepted row outputs d.
    * a rejected row outputs the oracle's residual winner, unless another
      token's score, with its residual raised by SPEC_REL_TOL p, comes within
      1e-6 of the winner's lowered score: then valid as above.
    ``gpu_p_at_token[b]`` is the GPU's p at its output token.
    """
    rep = SpecReport()
    B = len(orows)
    for b in range(B):
        rep.rows += 1
        o = orows[b]
        g, ga = int(gpu_token[b]), int(gpu_accepted[b])
        d = int(draft_token[b])

        def valid():
            if ga == 1:
                return g == d
            return 0 <= g < draft_probs.shape[1] and float(gpu_p_at_token[b]) > float(draft_probs[b, g])

        if o["status"] == 1:
            if g == -1 and ga == 0:
                rep.errors_ok += 1
            else:
                rep.failures.append((b, f"row error: gpu {g}/{ga}"))
            continue
        if int(gpu_keep_count[b]) != int(otarget["keep_count"][b]):
            t = otarget[b]
            p = float(top_p[b])
            in_band = bool(t["topp_active"]) and (abs(float(t["a_star"]) - p) <= MASS_BAND or
                                                 abs(float(t["m_star"]) - p) <= MASS_BAND)
            if not in_band:
                rep.failures.append((b, f"target keep count {int(gpu_keep_count[b])} vs oracle "
                                        f"{int(t['keep_count'])} outside the mass band"))
                continue
            rep.exempt_cut += 1
            if not valid():
                rep.failures.append((b, f"different cut: gpu output {g}/{ga} not valid"))
            continue
        gap = abs(o["u"] * o["q_draft"] - o["p_draft"])
        if gap <= SPEC_REL_TOL * o["p_draft"] + 1e-12:
            rep.exempt_accept += 1
            if not valid():
                rep.failures.append((b, f"acceptance boundary: gpu output {g}/{ga} not valid"))
            continue
        if ga != int(o["accepted"]):
            rep.failures.append((b, f"acceptance: gpu {ga}, oracle {int(o['accepted'])} (gap {gap:.3g})"))
            continue
        if ga == 1:
            rep.accepted += 1
            if g == d:
                rep.exact += 1
            else:
                rep.failures.append((b, f"accepted but gpu token {g} != draft {d}"))
            continue
        if o["status"] == 2:
            if g == -1:
                rep.exact += 1
            else:
                rep.failures.append((b, f"nothing to resample, gpu token {g}"))
            continue
        if o["threat"] * (1 + 1e-6) >= o["s1_low"] * (1 - 1e-6):
            rep.exempt_race += 1
            if not valid():
                rep.failures.append((b, f"race boundary: gpu output {g} not valid"))
            continue
        if g == int(o["token"]):
            rep.exact += 1
        else:
            rep.failures.append((b, f"residual draw: gpu {g}, oracle {int(o['token'])}"))
    return rep
