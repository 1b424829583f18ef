/*
 * nucleus_oracle.c -- plain float64 CPU reference ("the oracle") for batched
 * top-p (nucleus) sampling with per-row temperature, min-p, top-k and p.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU library is
 * measured against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  The GPU library never links, calls or reads
 * anything here, and nothing here is derived from the GPU code: the two share
 * no source, header, table or constant generator.
 *
 * Everything is computed the slow, obvious way: a full stable sort of each
 * row, float64 softmax, float64 cumulative sums, glibc exp/log.  Steps follow
 * the pages in their own order:
 *
 *   temperature  -> "What do temperature, top-k and top-p each do ...",
 *                   "A strong answer" (the tempered-softmax equation): the
 *                   logits are divided by T before the softmax, after the
 *                   row max is subtracted ("Implement batched top-p sampling
 *                   with temperature", "Why each line is there", item 1).
 *   min-p        -> same page, reference sampler: drop a token whose
 *                   probability is below min_p times the top probability.
 *   top-k        -> same page, reference sampler and its edge-case note:
 *                   keep values >= the k-th largest, ties at the k-th value
 *                   survive.
 *   top-p        -> "Top-p (Nucleus) Sampling, in depth", "Batched top-p with
 *                   a different p per request", and "Implement batched top-p
 *                   sampling ...", "How to approach it": keep token i iff the
 *                   mass of tokens strictly more probable than i is below p;
 *                   the top token is always kept; p >= 1 keeps everything.
 *                   The mass is taken over the min-p/top-k survivors,
 *                   renormalised (the chain of the temperature/top-k/top-p
 *                   page's reference sampler, which recomputes p from the
 *                   masked logits before its top-p step).
 *   sample       -> temperature/top-k/top-p page, "A strong answer", last
 *                   paragraph: argmax of p_i / E_i with E_i ~ Exp(1) draws
 *                   exactly from p.  E_i = -ln(u_i) with u_i from one
 *                   Philox4x32-10 word per token (see oracle_philox4x32_10).
 *   greedy       -> "Implement batched top-p sampling ...", "A strong
 *                   answer" and "Why each line is there", item 4:
 *                   temperature <= 0 is argmax, lowest index on ties.
 *   NaN logits   -> "Top-p (Nucleus) Sampling, in depth", "Failure modes":
 *                   check for NaN and fail the request (a row error here).
 *
 * Readings where the pages are silent are listed beside the code that takes
 * them.  Parity of the Philox stream itself is not fixed by the pages; it is
 * pinned against an independent library implementation in the tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Per-row result and the diagnostics the parity comparison needs. */
typedef struct {
    int32_t status;        /* 0 = ok, 1 = row error (NaN/+inf logit, NaN param, no finite logit) */
    int32_t token;         /* sampled id; -1 on row error */
    int32_t keep_count;    /* |Keep|; 0 on row error */
    int32_t n_survivors;   /* tokens left after min-p and top-k */
    int32_t greedy;        /* 1 when T <= 0 */
    int32_t topp_active;   /* 1 when 0 <= ... p < 1 decided the cut */
    double min_kept_logit; /* smallest kept logit; NaN on row error */
    double s_keep;         /* sum of e over Keep, e = exp((x - max)/T) */
    double s_surv;         /* sum of e over survivors */
    double a_star;         /* survivor-normalised mass strictly above the last kept level */
    double m_star;         /* a_star plus that level's mass = mass above the first dropped level */
    double race_s1;        /* best race score e_i/E_i */
    double race_s2;        /* second-best race score (0 if |Keep| == 1) */
    double race_margin;    /* (s1 - s2)/s1, 1 when |Keep| == 1 */
    double minp_nearest;   /* min over finite i of |p_i/(min_p*p_max) - 1|; +inf when min-p is off */
} oracle_row;

/* Evaluation of a caller-chosen cut (used to judge rows that sit on a boundary). */
typedef struct {
    int32_t status;
    int32_t token;         /* race winner over {survivor i : x_i >= cut} */
    int32_t keep_count;
    int32_t pad;
    double a_cut;          /* survivor-normalised mass strictly above the level x == cut */
    double m_cut;          /* a_cut plus the mass of the level x == cut */
    double s_keep;
    double race_s1;        /* oracle score of the winner */
} oracle_cut_eval;

/* ------------------------------------------------------------------------ */
/* Philox4x32-10, written from its published definition (Salmon, Moraes,     */
/* Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):         */
/* a 4-word counter and 2-word key; each round multiplies counter words 0 and */
/* 2 by the two round multipliers, and the new state is                      */
/*   (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));     */
/* the key is advanced by the two Weyl constants between rounds; 10 rounds.   */
/* ------------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The noise word of token i in row b.  Reading adopted (the pages only say
 * "exponential noise"; the key/counter layout is this library's contract):
 * key = (low, high 32 bits of seed); counter = (i / 4, b, low, high 32 bits
 * of step); token i takes output word i mod 4. */
uint32_t oracle_noise_word(uint64_t seed, uint64_t step, int64_t row, int64_t token)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {(uint32_t)(token >> 2), (uint32_t)row, (uint32_t)step, (uint32_t)(step >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[token & 3];
}

/* The noise words of tokens 0 .. n-1 of one row, word i at out[i]: the same
 * words oracle_noise_word gives one at a time (tests use it to place tokens
 * whose noise has a chosen property). */
void oracle_noise_words(uint64_t seed, uint64_t step, int64_t row, int64_t n, uint32_t* out)
{
    for (int64_t i = 0; i < n; i += 4) {
        uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
        uint32_t ctr[4] = {(uint32_t)(i >> 2), (uint32_t)row, (uint32_t)step, (uint32_t)(step >> 32)};
        uint32_t w[4];
        oracle_philox4x32_10(ctr, key, w);
        for (int j = 0; j < 4 && i + j < n; ++j) out[i + j] = w[j];
    }
}

/* Exp(1) variate from a word: u = (r + 1/2) / 2^32 lies strictly inside (0,1)
 * and is exact in double; E = -ln u. */
double oracle_exp1(uint32_t r)
{
    double u = ((double)r + 0.5) * (1.0 / 4294967296.0);
    return -log(u);
}

/* ------------------------------------------------------------------------ */
/* Row helpers                                                               */
/* ------------------------------------------------------------------------ */
static double widen(const void* logits, int dtype, int64_t off)
{
    if (dtype == ORACLE_BF16) {
        uint16_t h;
        memcpy(&h, (const unsigned char*)logits + 2 * off, 2);
        uint32_t bits = (uint32_t)h << 16;  /* bf16 is the top half of an fp32 */
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    float f;
    memcpy(&f, (const unsigned char*)logits + 4 * off, 4);
    return (double)f;
}

typedef struct {
    double v;
    int64_t i;
} vi_pair;

/* Descending by value, ascending index among equal values: the order a stable
 * descending sort produces. -0.0 and +0.0 compare equal (numeric ties). */
static int cmp_desc_stable(const void* a, const void* b)
{
    const vi_pair* x = (const vi_pair*)a;
    const vi_pair* y = (const vi_pair*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

/*
 * Top-p on one set of weighted items, from the definition: sort by `order`
 * descending (stable), normalise `mass` by its total, take the cumulative sum
 * in that order; a level (maximal run of equal `order`) is kept iff the
 * normalised mass strictly before it is < p; the first level is always kept;
 * p >= 1 keeps everything.  Writes keep[] in the caller's item order and
 * returns the number kept.  *a_star / *m_star receive the normalised mass
 * above the last kept level and above the first dropped level (NaN for p >= 1).
 *
 * Exported so that tests can pin the rule on the pages' probability-level
 * examples, where order == mass == the printed probabilities.
 */
int64_t oracle_topp_levels(const double* order, const double* mass, int64_t n, double p,
                           uint8_t* keep, double* a_star, double* m_star)
{
    if (a_star) *a_star = NAN;
    if (m_star) *m_star = NAN;
    if (n <= 0) return 0;
    if (p >= 1.0) {
        for (int64_t j = 0; j < n; ++j) keep[j] = 1;
        return n;
    }
    vi_pair* s = (vi_pair*)malloc((size_t)n * sizeof(vi_pair));
    for (int64_t j = 0; j < n; ++j) { s[j].v = order[j]; s[j].i = j; }
    qsort(s, (size_t)n, sizeof(vi_pair), cmp_desc_stable);

    double total = 0.0;
    for (int64_t j = 0; j < n; ++j) total += mass[s[j].i];

    for (int64_t j = 0; j < n; ++j) keep[j] = 0;
    int64_t kept = 0;
    double cum = 0.0;          /* running cumsum of the normalised mass in sorted order */
    int64_t j = 0;
    int first = 1;
    while (j < n) {
        int64_t lvl_end = j;   /* one past the level's last position */
        while (lvl_end < n && s[lvl_end].v == s[j].v) ++lvl_end;
        double a = cum;        /* mass strictly more probable than this level */
        if (!(first || a < p))
            break;             /* the cumsum only grows: every later level is dropped too */
        for (int64_t t = j; t < lvl_end; ++t) {
            keep[s[t].i] = 1;
            cum += mass[s[t].i] / total;
        }
        kept += lvl_end - j;
        if (a_star) *a_star = a;
        if (m_star) *m_star = cum;
        first = 0;
        j = lvl_end;
    }
    free(s);
    return kept;
}

/* Shared per-row preparation: validation, weights, min-p and top-k survivors. */
typedef struct {
    int err;
    int greedy;
    int64_t greedy_token;
    double m;          /* max finite logit */
    double* x;         /* widened logits */
    double* e;         /* exp((x - m)/T) for finite x, else 0 */
    uint8_t* surv;     /* min-p and top-k survivors */
    int64_t n_surv;
    double minp_nearest;
} row_prep;

static void prep_free(row_prep* r)
{
    free(r->x); free(r->e); free(r->surv);
    r->x = NULL; r->e = NULL; r->surv = NULL;
}

static void prep_row(const void* logits, int dtype, int64_t V, int64_t base, float T, float P,
                     int32_t K, float MP, row_prep* r)
{
    memset(r, 0, sizeof(*r));
    r->minp_nearest = INFINITY;
    r->x = (double*)malloc((size_t)V * sizeof(double));
    r->e = (double*)calloc((size_t)V, sizeof(double));
    r->surv = (uint8_t*)calloc((size_t)V, 1);

    /* 1. Validate: NaN or +inf logits, NaN parameters, no finite logit. */
    int64_t n_finite = 0;
    double m = -INFINITY;
    int64_t argmax = -1;
    for (int64_t i = 0; i < V; ++i) {
        double x = widen(logits, dtype, base + i);
        r->x[i] = x;
        if (isnan(x) || x == INFINITY) r->err = 1;
        if (x > -INFINITY && !isnan(x)) {
            ++n_finite;
            if (x > m) { m = x; argmax = i; }   /* strict '>' keeps the lowest index */
        }
    }
    if (isnan(T) || isnan(P) || isnan(MP) || n_finite == 0) r->err = 1;
    if (r->err) return;
    r->m = m;

    /* 2. Greedy: T <= 0 is argmax with the lowest index on ties. */
    if (T <= 0.0f) {
        r->greedy = 1;
        r->greedy_token = argmax;
        return;
    }

    /* 3. Tempered weights relative to the row max (softmax numerators). */
    double Td = (double)T;
    double total = 0.0;
    for (int64_t i = 0; i < V; ++i)
        if (r->x[i] > -INFINITY) { r->e[i] = exp((r->x[i] - m) / Td); total += r->e[i]; }

    /* 4. min-p: drop a token iff p_i < min_p * p_max.  min_p <= 0 is off;
     * min_p > 1 is clamped to 1 (reading: only the top level survives). */
    double mp = (double)MP;
    if (mp > 1.0) mp = 1.0;
    double pmax = 1.0 / total;     /* the max logit has e = 1 */
    for (int64_t i = 0; i < V; ++i) {
        if (!(r->x[i] > -INFINITY)) continue;
        double pi = r->e[i] / total;
        if (mp > 0.0) {
            r->surv[i] = !(pi < mp * pmax);
            double ratio = fabs(pi / (mp * pmax) - 1.0);
            if (ratio < r->minp_nearest) r->minp_nearest = ratio;
        } else {
            r->surv[i] = 1;
        }
    }

    /* 5. top-k: keep survivors whose logit is >= the k-th largest survivor
     * logit (ties at the k-th value survive); k <= 0 is off; k >= the number of
     * survivors is a no-op. */
    int64_t ns = 0;
    for (int64_t i = 0; i < V; ++i) ns += r->surv[i];
    if (K > 0 && (int64_t)K < ns) {
        vi_pair* s = (vi_pair*)malloc((size_t)ns * sizeof(vi_pair));
        int64_t t = 0;
        for (int64_t i = 0; i < V; ++i)
            if (r->surv[i]) { s[t].v = r->x[i]; s[t].i = i; ++t; }
        qsort(s, (size_t)ns, sizeof(vi_pair), cmp_desc_stable);
        double kth = s[K - 1].v;
        for (int64_t i = 0; i < V; ++i)
            if (r->surv[i] && r->x[i] < kth) r->surv[i] = 0;
        free(s);
    }
    r->n_surv = 0;
    for (int64_t i = 0; i < V; ++i) r->n_surv += r->surv[i];
}

/* The exponential race over a keep set: argmax e_i / E_i, lowest index among
 * equal maxima.  Returns the token; writes the best and second-best scores. */
static int64_t race(const row_prep* r, const uint8_t* keep, int64_t V, uint64_t seed, uint64_t step,
                    int64_t row, double* s1, double* s2)
{
    int64_t best = -1;
    double b1 = -1.0, b2 = -1.0;
    for (int64_t i = 0; i < V; ++i) {
        if (!keep[i]) continue;
        double E = oracle_exp1(oracle_noise_word(seed, step, row, i));
        double s = r->e[i] / E;
        if (s > b1) { b2 = b1; b1 = s; best = i; }
        else if (s > b2) { b2 = s; }
    }
    *s1 = b1;
    *s2 = b2 < 0.0 ? 0.0 : b2;
    return best;
}

/*
 * Sample rows [r0, r1) of a [B, V] batch (row b starts at element b*stride).
 * rows_out[b] receives the result of row b.  probs_out, if not NULL, is a
 * [r1 - r0, V] float64 array whose row (b - r0) receives the renormalised kept
 * distribution of row b (one-hot for greedy rows, zeros for error rows).
 * seeds, if not NULL, gives row b its own race key seeds[b] in place of seed
 * (a per-request seed; "Top-p (Nucleus) Sampling, in depth", "Logprobs,
 * speculative decoding and reproducibility").  logprobs_out, if not NULL, is
 * laid out like probs_out and receives the log-probabilities of the same
 * processed distribution (the same section: outside the nucleus the
 * probability is zero): ln p_i = (x_i - m)/T - ln S_keep for kept tokens, taken
 * in the log domain so that a kept token whose weight underflows stays finite;
 * -inf for every other token; 0 and -inf for greedy rows; NaN for error rows.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_sample_ex(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride,
                     const float* temperature, const float* top_p, const int32_t* top_k,
                     const float* min_p, uint64_t seed, const uint64_t* seeds, uint64_t step, int64_t r0,
                     int64_t r1, oracle_row* rows_out, double* probs_out, double* logprobs_out)
{
    if (V < 1 || B < 0 || r0 < 0 || r1 > B || stride < V || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return -1;
    for (int64_t b = r0; b < r1; ++b) {
        oracle_row* o = &rows_out[b];
        memset(o, 0, sizeof(*o));
        o->a_star = NAN; o->m_star = NAN; o->min_kept_logit = NAN;
        o->minp_nearest = INFINITY;
        double* prow = probs_out ? probs_out + (b - r0) * V : NULL;
        if (prow) memset(prow, 0, (size_t)V * sizeof(double));
        double* lrow = logprobs_out ? logprobs_out + (b - r0) * V : NULL;
        if (lrow)
            for (int64_t i = 0; i < V; ++i) lrow[i] = -INFINITY;
        const uint64_t row_seed = seeds ? seeds[b] : seed;

        float T = temperature[b], P = top_p[b], MP = min_p ? min_p[b] : 0.0f;
        int32_t K = top_k ? top_k[b] : 0;
        row_prep r;
        prep_row(logits, dtype, V, b * stride, T, P, K, MP, &r);
        if (r.err) {
            o->status = 1; o->token = -1; o->keep_count = 0;
            if (lrow)
                for (int64_t i = 0; i < V; ++i) lrow[i] = NAN;
            prep_free(&r);
            continue;
        }
        if (r.greedy) {
            o->greedy = 1;
            o->token = (int32_t)r.greedy_token;
            o->keep_count = 1;
            o->n_survivors = 1;
            o->min_kept_logit = r.x[r.greedy_token];
            o->s_keep = 1.0;
            o->race_margin = 1.0;
            if (prow) prow[r.greedy_token] = 1.0;
            if (lrow) lrow[r.greedy_token] = 0.0;
            prep_free(&r);
            continue;
        }
        o->minp_nearest = r.minp_nearest;
        o->n_survivors = (int32_t)r.n_surv;

        /* 6. top-p over the survivors, renormalised. */
        int64_t ns = r.n_surv;
        double* ord = (double*)malloc((size_t)ns * sizeof(double));
        double* ms = (double*)malloc((size_t)ns * sizeof(double));
        int64_t* id = (int64_t*)malloc((size_t)ns * sizeof(int64_t));
        uint8_t* kp = (uint8_t*)malloc((size_t)ns);
        int64_t t = 0;
        for (int64_t i = 0; i < V; ++i)
            if (r.surv[i]) { ord[t] = r.x[i]; ms[t] = r.e[i]; id[t] = i; ++t; }
        double Pd = (double)P;
        o->topp_active = Pd < 1.0;
        int64_t kept = oracle_topp_levels(ord, ms, ns, Pd, kp, &o->a_star, &o->m_star);
        for (int64_t j = 0; j < ns; ++j) o->s_surv += ms[j];

        uint8_t* keep = (uint8_t*)calloc((size_t)V, 1);
        double minkept = INFINITY;
        for (int64_t j = 0; j < ns; ++j)
            if (kp[j]) { keep[id[j]] = 1; if (ord[j] < minkept) minkept = ord[j]; }

        /* 7. Outputs: count, renormalised probabilities, smallest kept logit. */
        double s_keep = 0.0;
        for (int64_t i = 0; i < V; ++i) if (keep[i]) s_keep += r.e[i];
        o->keep_count = (int32_t)kept;
        o->s_keep = s_keep;
        o->min_kept_logit = minkept;
        if (prow)
            for (int64_t i = 0; i < V; ++i) prow[i] = keep[i] ? r.e[i] / s_keep : 0.0;
        if (lrow) {
            const double lse = log(s_keep), Td = (double)temperature[b];
            for (int64_t i = 0; i < V; ++i)
                if (keep[i]) lrow[i] = (r.x[i] - r.m) / Td - lse;
        }

        /* 8. The race. */
        double s1, s2;
        o->token = (int32_t)race(&r, keep, V, row_seed, step, b, &s1, &s2);
        o->race_s1 = s1;
        o->race_s2 = s2;
        o->race_margin = (kept <= 1) ? 1.0 : (s1 - s2) / s1;

        free(ord); free(ms); free(id); free(kp); free(keep);
        prep_free(&r);
    }
    return 0;
}

/* oracle_sample_ex with one seed for every row and no log-probabilities. */
int oracle_sample(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride,
                  const float* temperature, const float* top_p, const int32_t* top_k,
                  const float* min_p, uint64_t seed, uint64_t step, int64_t r0, int64_t r1,
                  oracle_row* rows_out, double* probs_out)
{
    return oracle_sample_ex(logits, dtype, B, V, stride, temperature, top_p, top_k, min_p, seed, NULL, step,
                            r0, r1, rows_out, probs_out, NULL);
}

/*
 * Judge a cut chosen elsewhere: with the oracle's own survivors of row b,
 * keep {i : x_i >= cut}, and report the mass above that cut's level, the
 * level's mass (both normalised over the survivors), the race winner over
 * that keep set and its count.  probs_row (nullable, [V]) receives the
 * renormalised probabilities of that keep set.  Returns 0, or -1 on bad
 * arguments; status 1 for a row error; greedy rows are not meaningful here.
 */
int oracle_eval_cut(const void* logits, int dtype, int64_t V, int64_t row_offset, int64_t row,
                    float temperature, float top_p, int32_t top_k, float min_p, uint64_t seed,
                    uint64_t step, double cut, oracle_cut_eval* out, double* probs_row)
{
    (void)top_p;
    if (V < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    memset(out, 0, sizeof(*out));
    if (probs_row) memset(probs_row, 0, (size_t)V * sizeof(double));
    row_prep r;
    prep_row(logits, dtype, V, row_offset, temperature, top_p, top_k, min_p, &r);
    if (r.err || r.greedy) {
        out->status = r.err ? 1 : 2;
        out->token = -1;
        prep_free(&r);
        return 0;
    }
    double s_surv = 0.0, above = 0.0, level = 0.0;
    for (int64_t i = 0; i < V; ++i) if (r.surv[i]) s_surv += r.e[i];
    for (int64_t i = 0; i < V; ++i) {
        if (!r.surv[i]) continue;
        if (r.x[i] > cut) above += r.e[i];
        else if (r.x[i] == cut) level += r.e[i];
    }
    out->a_cut = above / s_surv;
    out->m_cut = (above + level) / s_surv;
    uint8_t* keep = (uint8_t*)calloc((size_t)V, 1);
    int64_t kept = 0;
    double s_keep = 0.0;
    for (int64_t i = 0; i < V; ++i)
        if (r.surv[i] && r.x[i] >= cut) { keep[i] = 1; ++kept; s_keep += r.e[i]; }
    out->keep_count = (int32_t)kept;
    out->s_keep = s_keep;
    if (probs_row && kept)
        for (int64_t i = 0; i < V; ++i) probs_row[i] = keep[i] ? r.e[i] / s_keep : 0.0;
    if (kept) {
        double s1, s2;
        out->token = (int32_t)race(&r, keep, V, seed, step, row, &s1, &s2);
        out->race_s1 = s1;
    } else {
        out->token = -1;
    }
    free(keep);
    prep_free(&r);
    return 0;
}

/* Oracle score e_i / E_i of token i of row b (for judging near-tied races). */
double oracle_race_score(const void* logits, int dtype, int64_t V, int64_t row_offset, int64_t row,
                         float temperature, uint64_t seed, uint64_t step, int64_t token)
{
    double m = -INFINITY;
    for (int64_t i = 0; i < V; ++i) {
        double x = widen(logits, dtype, row_offset + i);
        if (x > m) m = x;
    }
    double x = widen(logits, dtype, row_offset + token);
    double e = exp((x - m) / (double)temperature);
    return e / oracle_exp1(oracle_noise_word(seed, step, row, token));
}

/* ------------------------------------------------------------------------ */
/* Sort-free top-p by rejection ("Top-p (Nucleus) Sampling, in depth",       */
/* "Sort-free top-p by rejection sampling"): a second way to draw from the   */
/* same kept distribution, with no sort and no cut.                          */
/* ------------------------------------------------------------------------ */

/* Result of the rejection sampler for one row. */
typedef struct {
    int32_t status;      /* 0 = ok, 1 = row error, 2 = no token accepted within max_rounds */
    int32_t token;       /* accepted id; -1 on a row error or with no acceptance */
    int32_t rounds;      /* proposal rounds run (0 for greedy and error rows) */
    int32_t greedy;      /* 1 when T <= 0 */
    double band;         /* min over the rounds' acceptance tests of |A(t)/S - p| (+inf if none was close) */
    double race_margin;  /* min over the rounds' proposal races of (s1 - s2)/s1 (1 for a lone proposal) */
} oracle_rej_row;

/*
 * Rows [r0, r1) of a [B, V] batch by rejection.  Per row, with the same
 * validation, greedy rule, weights e_i and min-p survivors as oracle_sample
 * (top-k is not part of this variant), S = sum of e over the survivors:
 *
 *   the pivot starts below every logit.  Round r draws a proposal t among
 *   the finite tokens strictly above the pivot, with probability
 *   proportional to e: the exponential race argmax e_i / E_i over them,
 *   lowest index on ties, with the row's noise words E_i (the same words as
 *   oracle_sample).  t is accepted iff it survives min-p and either it is in
 *   the top level (always kept), or p >= 1 (every survivor is kept), or
 *   p > 0 and the survivor mass strictly above it, A(t), is below p S (the
 *   order-free top-p rule; p <= 0 keeps the top level only).  Otherwise t and every token at or below it are out: the
 *   pivot becomes x_t and the next round draws again.
 *
 * Reusing the words in every round is a valid draw: in arrival-time form
 * (token i arrives at E_i / e_i, exponential with rate e_i) the race's
 * winner is the first arrival, and given that the first arrivals so far were
 * rejected tokens, the remaining tokens' waiting times are again independent
 * exponentials with the same rates (memorylessness), so each round's
 * proposal is proportional to e among the tokens above the pivot.  It also
 * means the accepted token is the first kept token to arrive: exactly
 * oracle_sample's token.  The kept set is a top set of levels above every
 * pivot, and every round raises the pivot, so a row needs at most one round
 * per distinct level.  rows_out[b] receives row b's result.  Returns 0, or
 * -1 on bad arguments.
 */
int oracle_sample_rejection(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride,
                            const float* temperature, const float* top_p, const float* min_p, uint64_t seed,
                            const uint64_t* seeds, uint64_t step, int32_t max_rounds, int64_t r0, int64_t r1,
                            oracle_rej_row* rows_out)
{
    if (V < 1 || B < 0 || r0 < 0 || r1 > B || stride < V || max_rounds < 1 ||
        (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return -1;
    uint8_t* prop = (uint8_t*)malloc((size_t)V);
    for (int64_t b = r0; b < r1; ++b) {
        oracle_rej_row* o = &rows_out[b];
        memset(o, 0, sizeof(*o));
        o->band = INFINITY;
        o->race_margin = 1.0;
        const uint64_t key = seeds ? seeds[b] : seed;  /* the row's race key */
        const float T = temperature[b], P = top_p[b], MP = min_p ? min_p[b] : 0.0f;
        row_prep r;
        prep_row(logits, dtype, V, b * stride, T, P, 0, MP, &r);
        if (r.err) {
            o->status = 1;
            o->token = -1;
            prep_free(&r);
            continue;
        }
        if (r.greedy) {
            o->greedy = 1;
            o->token = (int32_t)r.greedy_token;
            prep_free(&r);
            continue;
        }
        double S = 0.0;
        for (int64_t i = 0; i < V; ++i)
            if (r.surv[i]) S += r.e[i];
        const double Pd = (double)P;
        double pivot = -INFINITY;
        o->status = 2;
        o->token = -1;
        o->rounds = max_rounds;
        for (int32_t round = 1; round <= max_rounds; ++round) {
            int64_t n_prop = 0;
            for (int64_t i = 0; i < V; ++i) {
                prop[i] = r.x[i] > -INFINITY && r.x[i] > pivot;
                n_prop += prop[i];
            }
            double s1, s2;
            const int64_t t = race(&r, prop, V, key, step, b, &s1, &s2);
            const double margin = n_prop > 1 ? (s1 - s2) / s1 : 1.0;
            if (margin < o->race_margin) o->race_margin = margin;
            const double xt = r.x[t];
            double A = 0.0;
            for (int64_t i = 0; i < V; ++i)
                if (r.surv[i] && r.x[i] > xt) A += r.e[i];
            int accept = 0;
            if (r.surv[t]) {
                if (xt == r.m || Pd >= 1.0) {  /* p >= 1 keeps every survivor, however light */
                    accept = 1;
                } else if (Pd > 0.0) {
                    accept = A < Pd * S;
                    const double d = fabs(A / S - Pd);
                    if (d < o->band) o->band = d;
                }
            }
            if (accept) {
                o->status = 0;
                o->token = (int32_t)t;
                o->rounds = round;
                break;
            }
            pivot = xt;
        }
        prep_free(&r);
    }
    free(prop);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Speculative-decoding acceptance ("Top-p (Nucleus) Sampling, in depth",    */
/* "Logprobs, speculative decoding and reproducibility"): a draft token d    */
/* drawn from the draft's distribution q is accepted with probability        */
/* min(1, p(d)/q(d)); otherwise the token is drawn from the normalised       */
/* positive part of p - q.  p is the target's truncated, renormalised        */
/* distribution (the kept set of oracle_sample), never the raw softmax.      */
/* ------------------------------------------------------------------------ */

/* Noise of the verification step (reading adopted; the pages fix none): the
 * Philox key of the row, counter word 1 = row index with bit 31 set (so the
 * words never repeat nucleus_sample's race words for the same seed and
 * step), words 2-3 = step.  Token i of the residual draw takes word i mod 4 of
 * counter word 0 = i / 4; the acceptance uniform is word 0 at counter word
 * 0 = 0xFFFFFFFF, which no token reaches (i / 4 < 2^29). */
static uint32_t spec_word(uint64_t key, uint64_t step, int64_t row, uint32_t c0, int word)
{
    uint32_t k[2] = {(uint32_t)key, (uint32_t)(key >> 32)};
    uint32_t ctr[4] = {c0, (uint32_t)row | 0x80000000u, (uint32_t)step, (uint32_t)(step >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, k, out);
    return out[word];
}

typedef struct {
    int32_t status;     /* 0 = ok, 1 = target row error or draft token out of range, 2 = nothing to resample */
    int32_t token;      /* output token; -1 unless status 0 */
    int32_t accepted;   /* 1 when the draft token was accepted */
    int32_t greedy;     /* 1 when the target row is greedy (p one-hot) */
    double p_draft;     /* p(d), q(d) and the acceptance uniform u */
    double q_draft;
    double u;
    double s1;          /* winning residual score r_i / E_i (rejections) */
    double s1_low;      /* that score with the winner's residual lowered by tol */
    double threat;      /* best score another token reaches with its residual raised by tol */
} oracle_spec_row;

/*
 * Verify rows [r0, r1): target logits and chain parameters as for
 * oracle_sample (row b's kept distribution p), draft distribution q
 * ([B, V] float, row-major) and draft tokens d[B].  With u the acceptance
 * uniform, the draft is accepted iff u q(d) < p(d) (probability
 * min(1, p(d)/q(d)); q(d) = 0 accepts iff p(d) > 0).  Otherwise the token is
 * the exponential race argmax_i r_i / E_i over r_i = max(0, p_i - q_i) > 0,
 * lowest index on ties: a draw from the normalised residual.  The accepted
 * or resampled token then follows p exactly, whatever q is.
 *
 * For judging a GPU that holds p to within tol_i = rel_tol p_i on kept tokens
 * (exactly 0 elsewhere), s1_low and threat bound the race under that
 * uncertainty.  Returns 0, or -1 on bad arguments.
 */
int oracle_spec_verify(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride,
                       const float* temperature, const float* top_p, const int32_t* top_k, const float* min_p,
                       const float* draft_probs, const int32_t* draft_token, uint64_t seed, const uint64_t* seeds,
                       uint64_t step, double rel_tol, int64_t r0, int64_t r1, oracle_spec_row* rows_out)
{
    if (V < 1 || B < 0 || r0 < 0 || r1 > B || stride < V || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return -1;
    double* p = (double*)malloc((size_t)V * sizeof(double));
    oracle_row* target = (oracle_row*)calloc((size_t)B, sizeof(oracle_row));
    for (int64_t b = r0; b < r1; ++b) {
        oracle_spec_row* o = &rows_out[b];
        memset(o, 0, sizeof(*o));
        o->token = -1;
        /* The target's kept, renormalised distribution of row b. */
        oracle_sample_ex(logits, dtype, B, V, stride, temperature, top_p, top_k, min_p, seed, seeds, step, b, b + 1,
                         target, p, NULL);
        const oracle_row tr = target[b];
        const int32_t d = draft_token[b];
        if (tr.status != 0 || d < 0 || d >= V) {
            o->status = 1;
            continue;
        }
        o->greedy = tr.greedy;
        const uint64_t key = seeds ? seeds[b] : seed;
        const float* q = draft_probs + b * V;
        o->p_draft = p[d];
        o->q_draft = (double)q[d];
        o->u = ((double)spec_word(key, step, b, 0xFFFFFFFFu, 0) + 0.5) * (1.0 / 4294967296.0);
        if (o->u * o->q_draft < o->p_draft) {
            o->accepted = 1;
            o->token = d;
            continue;
        }
        int64_t best = -1;
        double s1 = -1.0, threat = 0.0;
        for (int64_t i = 0; i < V; ++i) {
            const double r = p[i] - (double)q[i];
            const double tol = rel_tol * p[i];
            if (!(r > 0.0) && !(r + tol > 0.0)) continue;
            const double E = oracle_exp1(spec_word(key, step, b, (uint32_t)(i >> 2), (int)(i & 3)));
            if (r > 0.0) {
                const double s = r / E;
                if (s > s1) {
                    if (best >= 0) {
                        const double up = (p[best] - (double)q[best] + rel_tol * p[best]) / oracle_exp1(
                            spec_word(key, step, b, (uint32_t)(best >> 2), (int)(best & 3)));
                        if (up > threat) threat = up;
                    }
                    s1 = s;
                    best = i;
                    continue;
                }
            }
            const double up = (r + tol) / E;
            if (up > threat) threat = up;
        }
        if (best < 0) {
            o->status = 2;
            continue;
        }
        o->token = (int32_t)best;
        o->s1 = s1;
        o->s1_low = (p[best] - (double)q[best] - rel_tol * p[best]) /
                    oracle_exp1(spec_word(key, step, b, (uint32_t)(best >> 2), (int)(best & 3)));
        o->threat = threat;
    }
    free(target);
    free(p);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The pre-chain ("Top-p (Nucleus) Sampling, in depth", "Where top-p sits in  */
/* the sampler chain"; "What do temperature, top-k and top-p ...", "What      */
/* interviewers probe next"): penalties on the raw logits, then the grammar   */
/* mask, before temperature and the filters.  The pages name the penalties   */
/* but give no formulas; the readings adopted are the common definitions:    */
/*                                                                          */
/*   c_i     = occurrences of token i in the row's history (duplicates count) */
/*   repetition (rho > 0, 1 = off), for c_i > 0:                             */
/*             x <- x / rho if x > 0, else x * rho                            */
/*   frequency (a_f) and presence (a_p), for c_i > 0, after repetition:       */
/*             x <- x - (a_f * c_i + a_p)                                     */
/*   mask    : token i allowed iff bit (i mod 32) of word i / 32 is set;      */
/*             a disallowed token becomes -inf (after the penalties)          */
/*                                                                          */
/* Every step is one IEEE float operation in the order written (no fused     */
/* multiply-add), so the processed logits are exact fp32 values any          */
/* implementation reproduces; the sampler then runs on them unchanged.       */
/* ------------------------------------------------------------------------ */
int oracle_preprocess(const void* logits, int dtype, int64_t B, int64_t V, int64_t stride, const int32_t* hist,
                      int64_t H, const float* repetition, const float* frequency, const float* presence,
                      const uint32_t* allowed, float* out)
{
    if (V < 1 || B < 0 || stride < V || H < 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return -1;
    const int64_t words = (V + 31) / 32;
    int32_t* count = (int32_t*)calloc((size_t)V, sizeof(int32_t));
    for (int64_t b = 0; b < B; ++b) {
        memset(count, 0, (size_t)V * sizeof(int32_t));
        for (int64_t h = 0; h < H && hist; ++h) {
            const int32_t tok = hist[b * H + h];
            if (tok >= 0 && tok < V) count[tok] += 1;  /* -1 pads; ids outside [0, V) are ignored */
        }
        const float rho = repetition ? repetition[b] : 1.0f;
        const float af = frequency ? frequency[b] : 0.0f;
        const float ap = presence ? presence[b] : 0.0f;
        for (int64_t i = 0; i < V; ++i) {
            float x = (float)widen(logits, dtype, b * stride + i);
            if (count[i] > 0) {
                volatile float y = x > 0.0f ? x / rho : x * rho;
                volatile float pen = af * (float)count[i];
                pen = pen + ap;
                x = y - pen;
            }
            if (allowed && !((allowed[b * words + i / 32] >> (i % 32)) & 1u)) x = -INFINITY;
            out[b * V + i] = x;
        }
    }
    free(count);
    return 0;
}
