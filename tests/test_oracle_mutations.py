"""Plant plausible mistakes in copies of the oracle's C source (on the CPU),
build each copy, and require the pins to reject every one of them.  This is
evidence that the pins constrain each step of the oracle: the boundary
comparison, the always-kept top level, greedy tie-breaking, the temperature,
min-p, top-k, renormalisation, validation, Philox, the race, the
rejection sampler, speculative acceptance, the pre-chain, and the judges of
boundary rows (oracle_eval_cut, oracle_race_score)."""
import os
import shutil

import pytest

import oracle
import oracle_pins as P

# (name, text in nucleus_oracle.c, replacement)
MUTATIONS = [
    ("boundary inclusive", "if (!(first || a < p))", "if (!(first || a <= p))"),
    ("top level not forced", "if (!(first || a < p))", "if (!(a < p))"),
    ("unshifted cumsum", "double a = cum;        /* mass strictly", "double a = cum + mass[s[j].i] / total; /*"),
    ("greedy highest index", "if (x > m) { m = x; argmax = i; }", "if (x >= m) { m = x; argmax = i; }"),
    ("temperature multiplies", "exp((r->x[i] - m) / Td)", "exp((r->x[i] - m) * Td)"),
    ("min-p without p_max", "r->surv[i] = !(pi < mp * pmax);", "r->surv[i] = !(pi < mp);"),
    ("top-k drops ties", "if (r->surv[i] && r->x[i] < kth)", "if (r->surv[i] && r->x[i] <= kth)"),
    ("top-k off by one", "double kth = s[K - 1].v;", "double kth = s[K].v;"),
    ("renormalise by survivors", "prow[i] = keep[i] ? r.e[i] / s_keep : 0.0;", "prow[i] = keep[i] ? r.e[i] / o->s_surv : 0.0;"),
    ("+inf accepted", "if (isnan(x) || x == INFINITY) r->err = 1;", "if (isnan(x)) r->err = 1;"),
    ("race multiplies noise", "double s = r->e[i] / E;", "double s = r->e[i] * E;"),
    ("philox weyl constant", "W0 = 0x9E3779B9u", "W0 = 0x9E3779B7u"),
    ("philox word order", "return out[token & 3];", "return out[3 - (token & 3)];"),
    ("philox counter layout", "uint32_t ctr[4] = {(uint32_t)(token >> 2), (uint32_t)row,",
     "uint32_t ctr[4] = {(uint32_t)row, (uint32_t)(token >> 2),"),
    ("uniform off by half", "double u = ((double)r + 0.5)", "double u = ((double)r + 1.0)"),
    ("logprob not normalised", "if (keep[i]) lrow[i] = (r.x[i] - r.m) / Td - lse;",
     "if (keep[i]) lrow[i] = (r.x[i] - r.m) / Td;"),
    ("logprob untempered", "if (keep[i]) lrow[i] = (r.x[i] - r.m) / Td - lse;",
     "if (keep[i]) lrow[i] = (r.x[i] - r.m) - lse;"),
    ("logprob of every survivor", "if (keep[i]) lrow[i] = (r.x[i] - r.m) / Td - lse;",
     "if (r.surv[i]) lrow[i] = (r.x[i] - r.m) / Td - lse;"),
    ("row seed ignored", "const uint64_t row_seed = seeds ? seeds[b] : seed;", "const uint64_t row_seed = seed;"),
    ("rejection pivot inclusive", "prop[i] = r.x[i] > -INFINITY && r.x[i] > pivot;",
     "prop[i] = r.x[i] > -INFINITY && r.x[i] >= pivot;"),
    ("rejection mass includes the level", "if (r.surv[i] && r.x[i] > xt) A += r.e[i];",
     "if (r.surv[i] && r.x[i] >= xt) A += r.e[i];"),
    ("rejection top level not forced", "if (xt == r.m || Pd >= 1.0) {", "if (Pd >= 1.0) {"),
    ("rejection min-p ignored", "if (r.surv[t]) {", "if (1) {"),
    ("rejection total over all tokens", "if (r.surv[i]) S += r.e[i];", "S += r.e[i];"),
    ("rejection pivot not raised", "pivot = xt;", "pivot = -INFINITY;"),
    ("speculative acceptance reversed", "if (o->u * o->q_draft < o->p_draft) {", "if (o->u * o->p_draft < o->q_draft) {"),
    ("speculative acceptance ignores q", "if (o->u * o->q_draft < o->p_draft) {", "if (o->u < o->p_draft) {"),
    ("speculative residual reversed", "const double r = p[i] - (double)q[i];", "const double r = (double)q[i] - p[i];"),
    ("repetition divides negative logits", "volatile float y = x > 0.0f ? x / rho : x * rho;",
     "volatile float y = x / rho;"),
    ("duplicates counted once", "if (tok >= 0 && tok < V) count[tok] += 1;", "if (tok >= 0 && tok < V) count[tok] = 1;"),
    ("presence per occurrence", "pen = pen + ap;", "pen = pen + ap * (float)count[i];"),
    ("judge mass over every finite token", "        if (!r.surv[i]) continue;\n        if (r.x[i] > cut) above += r.e[i];",
     "        if (!(r.x[i] > -INFINITY)) continue;\n        if (r.x[i] > cut) above += r.e[i];"),
    ("judge mass above inclusive", "if (r.x[i] > cut) above += r.e[i];", "if (r.x[i] >= cut) above += r.e[i];"),
    ("judge keeps only above the cut", "if (r.surv[i] && r.x[i] >= cut) { keep[i] = 1;",
     "if (r.surv[i] && r.x[i] > cut) { keep[i] = 1;"),
    ("race score without the row max", "double e = exp((x - m) / (double)temperature);",
     "double e = exp(x / (double)temperature);"),
    ("mask bits reversed", "(allowed[b * words + i / 32] >> (i % 32)) & 1u", "(allowed[b * words + i / 32] >> (31 - i % 32)) & 1u"),
]


def _checks(tmp, need_rocrand):
    checks = list(P.ALL_FAST_CHECKS) + [
        lambda O: P.check_bruteforce_protocol(O, batches=300, seed=11, extras=True),
        P.check_race_frequencies,
    ]
    if need_rocrand:
        tuples = P.philox_tuples(200)
        words = P.rocrand_words(tuples, tmp)
        checks.append(lambda O: P.check_philox_against(O, tuples, words))
    return checks


def _fails(O, checks):
    for c in checks:
        try:
            c(O)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_every_planted_mistake_is_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "nucleus_oracle.c")).read()
    checks = _checks(str(tmp_path), shutil.which("hipcc") is not None)
    # The unmodified source passes.
    assert not _fails(oracle.default(), checks)
    survivors = []
    for j, (name, old, new) in enumerate(MUTATIONS):
        assert src.count(old) == 1, name
        path = tmp_path / f"m{j}.c"
        path.write_text(src.replace(old, new))
        lib = oracle.build(src=str(path), out=str(tmp_path / f"m{j}.so"))
        if not _fails(oracle.Oracle(lib), checks):
            survivors.append(name)
    assert not survivors, f"mutations not caught by any pin: {survivors}"
