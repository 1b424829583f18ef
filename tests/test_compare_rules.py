"""The parity harness itself (oracle/compare.py), on the CPU: each comparison
accepts the oracle's own results and rejects a planted wrong token, count,
cut, probability, round count or acceptance.  Without this, a comparison
that passed everything would make every GPU parity test vacuous."""
import numpy as np

import oracle
import workloads
from oracle.compare import SPEC_REL_TOL, compare, compare_rejection, compare_spec


def _batch():
    w = workloads.make(1)
    return w


def test_compare_accepts_the_oracle_and_rejects_mistakes():
    w = _batch()
    rows, probs = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"],
                                want_probs=True)
    tok = rows["token"].copy()
    cnt = rows["keep_count"].copy()
    mk = rows["min_kept_logit"].astype(np.float32)
    pr = probs.astype(np.float32)
    args = (w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], w["seed"], 0)
    ok = compare(*args, tok, cnt, mk, rows, gpu_probs=pr, oracle_probs=probs, prob_rows=list(range(w["B"])))
    assert ok.ok(), ok.failures
    b = int(np.nonzero((rows["greedy"] == 0) & (rows["keep_count"] > 2) & (rows["status"] == 0))[0][0])
    bad = tok.copy()
    bad[b] = (bad[b] + 1) % w["V"]
    assert not compare(*args, bad, cnt, mk, rows).ok()          # another token
    bad = cnt.copy()
    bad[b] += 1
    assert not compare(*args, tok, bad, mk, rows).ok()          # another count
    bad = mk.copy()
    bad[b] = np.nextafter(bad[b], np.float32(np.inf))
    assert not compare(*args, tok, cnt, bad, rows).ok()         # another cut
    bad = pr.copy()
    bad[b, tok[b]] *= 1.001
    assert not compare(*args, tok, cnt, mk, rows, gpu_probs=bad, oracle_probs=probs,
                       prob_rows=list(range(w["B"]))).ok()      # a probability off by 1e-3


def test_compare_rejection_accepts_the_oracle_and_rejects_mistakes():
    w = _batch()
    orows = oracle.sample_rejection(w["logits"], w["temperature"], w["top_p"], w["min_p"], seed=w["seed"])
    tok, rounds = orows["token"].copy(), orows["rounds"].copy()
    args = (w["logits"], w["temperature"], w["top_p"], w["min_p"], w["seed"], 0)
    assert compare_rejection(*args, tok, rounds, orows).ok()
    b = int(np.nonzero((orows["greedy"] == 0) & (orows["status"] == 0) & (orows["band"] > 1e-3))[0][0])
    bad = tok.copy()
    bad[b] = (bad[b] + 1) % w["V"]
    assert not compare_rejection(*args, bad, rounds, orows).ok()
    bad = rounds.copy()
    bad[b] += 1
    assert not compare_rejection(*args, tok, bad, orows).ok()


def test_compare_spec_accepts_the_oracle_and_rejects_mistakes():
    w = _batch()
    q, d = workloads.make_draft(w, seed=4)
    rows, probs = oracle.sample(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], seed=w["seed"],
                                want_probs=True)
    o = oracle.spec_verify(w["logits"], w["temperature"], w["top_p"], w["top_k"], w["min_p"], q, d, seed=w["seed"],
                           rel_tol=SPEC_REL_TOL)
    tok, acc = o["token"].copy(), o["accepted"].copy()
    p_at = probs[np.arange(w["B"]), np.clip(tok, 0, w["V"] - 1)]
    cnt = rows["keep_count"]
    assert compare_spec(q, d, tok, acc, cnt, p_at, o, rows, w["top_p"]).ok()
    clear = np.nonzero((o["status"] == 0) & (np.abs(o["u"] * o["q_draft"] - o["p_draft"]) > 1e-3))[0]
    b = int(clear[0])
    bad = acc.copy()
    bad[b] = 1 - bad[b]
    assert not compare_spec(q, d, tok, bad, cnt, p_at, o, rows, w["top_p"]).ok()     # the other acceptance
    rej = [int(r) for r in clear if o["accepted"][r] == 0 and o["threat"][r] < 0.5 * o["s1_low"][r]]
    if rej:
        r = rej[0]
        bad = tok.copy()
        bad[r] = d[r] if d[r] != tok[r] else (tok[r] + 1) % w["V"]
        assert not compare_spec(q, d, bad, acc, cnt, p_at, o, rows, w["top_p"]).ok()  # another residual draw
    # A different target cut on a row far from the mass band is a failure,
    # even when the output would be valid for that other cut.
    far = [int(r) for r in np.nonzero((rows["status"] == 0) & (rows["greedy"] == 0) & (rows["topp_active"] == 1))[0]
           if min(abs(rows["a_star"][r] - w["top_p"][r]), abs(rows["m_star"][r] - w["top_p"][r])) > 1e-3]
    r = far[0]
    bad = cnt.copy()
    bad[r] += 1
    assert not compare_spec(q, d, tok, acc, bad, p_at, o, rows, w["top_p"]).ok()  # another cut, outside the band
