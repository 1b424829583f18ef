/*
 * Drives every entry point of the oracle (oracle/nucleus_oracle.c, compiled
 * into this program) over small seeded batches that reach its edge cases:
 * NaN and +inf logits, rows with no finite logit, greedy, infinite and NaN
 * temperatures, p at 0, 1 and NaN, top-k of 1, beyond V and negative, min-p
 * at 0, 1 and NaN, bf16 rows, strided rows, per-row keys, histories with
 * out-of-range ids, zero draft probabilities, and bad arguments.  Built with
 * gcc -fsanitize=address,undefined -fno-sanitize-recover=all, so any
 * out-of-bounds access, leak, use after free, signed overflow, bad shift or
 * misaligned access aborts it.  Prints "ok" and returns 0 otherwise.
 *
 * TEST INFRASTRUCTURE ONLY.
 */
#include "../../oracle/nucleus_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x243F6A8885A308D3ull;

static uint64_t next_u64(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform01(void) { return (double)(next_u64() >> 11) * 0x1p-53; }

static float normal(void)
{
    double u1 = uniform01(), u2 = uniform01();
    if (u1 < 1e-300) u1 = 1e-300;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int failures = 0;

#define CHECK(c)                                                     \
    do {                                                             \
        if (!(c)) {                                                  \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                              \
        }                                                            \
    } while (0)

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN stays NaN */
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

enum { B = 24, V = 301, STRIDE = 307, H = 40 };

int main(void)
{
    float* x = (float*)malloc(sizeof(float) * B * STRIDE);
    uint16_t* xb = (uint16_t*)malloc(sizeof(uint16_t) * B * STRIDE);
    float T[B], P[B], MP[B];
    int32_t K[B];
    uint64_t seeds[B];
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < STRIDE; ++i) x[b * STRIDE + i] = i < V ? 2.0f * normal() : NAN; /* NaN padding: never read */
        T[b] = (float)(0.3 + 1.4 * uniform01());
        P[b] = (float)(0.2 + 0.79 * uniform01());
        K[b] = 0;
        MP[b] = 0.0f;
        seeds[b] = next_u64();
    }
    /* Edge rows. */
    x[0 * STRIDE + 5] = NAN;
    x[1 * STRIDE + 7] = INFINITY;
    for (int i = 0; i < V; ++i) x[2 * STRIDE + i] = -INFINITY;
    T[3] = 0.0f;
    T[4] = -1.0f;
    T[5] = INFINITY;
    T[6] = NAN;
    P[7] = 0.0f;
    P[8] = 1.0f;
    P[9] = NAN;
    K[10] = 1;
    K[11] = V + 5;
    K[12] = -3;
    K[13] = 17;
    MP[14] = 0.1f;
    MP[15] = 1.0f;
    MP[16] = NAN;
    MP[17] = 5.0f;
    for (int i = 0; i < V; ++i) x[18 * STRIDE + i] = (float)((i * 7) % 5); /* ties straddle the cut */
    for (int i = 0; i < V; ++i) x[19 * STRIDE + i] = 1e-40f * (float)(i % 3); /* subnormal logits */
    T[19] = 1e-38f;
    x[20 * STRIDE + 0] = 3e38f;
    x[20 * STRIDE + 1] = -3e38f;
    T[21] = 1e-30f;
    for (int i = 1; i < V; ++i) x[22 * STRIDE + i] = -INFINITY; /* one finite token */
    for (int i = 0; i < B * STRIDE; ++i) xb[i] = to_bf16(x[i]);

    oracle_row rows[B];
    double* probs = (double*)malloc(sizeof(double) * B * V);
    double* lps = (double*)malloc(sizeof(double) * B * V);
    for (int dt = 0; dt < 2; ++dt) {
        const void* lg = dt == ORACLE_F32 ? (const void*)x : (const void*)xb;
        for (int keyed = 0; keyed < 2; ++keyed) {
            CHECK(oracle_sample_ex(lg, dt, B, V, STRIDE, T, P, K, MP, 77, keyed ? seeds : NULL, 3, 0, B, rows, probs,
                                   lps) == 0);
            for (int b = 0; b < B; ++b) {
                if (rows[b].status != 0) {
                    CHECK(rows[b].token == -1);
                    continue;
                }
                CHECK(rows[b].token >= 0 && rows[b].token < V && rows[b].keep_count >= 1);
                double s = 0.0;
                for (int i = 0; i < V; ++i) s += probs[b * V + i];
                CHECK(fabs(s - 1.0) < 1e-9);
                CHECK(probs[b * V + rows[b].token] > 0.0);
            }
        }
        CHECK(oracle_sample(lg, dt, B, V, STRIDE, T, P, NULL, NULL, 5, 0, 3, 9, rows, NULL) == 0);
        /* Judges at the oracle's own cut and at a neighbouring one. */
        CHECK(oracle_sample_ex(lg, dt, B, V, STRIDE, T, P, K, MP, 77, NULL, 0, 0, B, rows, NULL, NULL) == 0);
        for (int b = 0; b < B; ++b) {
            oracle_cut_eval ev;
            double* pr = (double*)malloc(sizeof(double) * V);
            const double cut = rows[b].status == 0 ? rows[b].min_kept_logit : 0.0;
            CHECK(oracle_eval_cut(lg, dt, V, (int64_t)b * STRIDE, b, T[b], P[b], K[b], MP[b], 77, 0, cut, &ev, pr) == 0);
            CHECK(oracle_eval_cut(lg, dt, V, (int64_t)b * STRIDE, b, T[b], P[b], K[b], MP[b], 77, 0, cut + 0.25, &ev,
                                  NULL) == 0);
            (void)oracle_race_score(lg, dt, V, (int64_t)b * STRIDE, b, T[b], 77, 0, b % V);
            free(pr);
        }
        /* Rejection (top-k is not part of it) and speculative verification. */
        oracle_rej_row rj[B];
        CHECK(oracle_sample_rejection(lg, dt, B, V, STRIDE, T, P, MP, 9, NULL, 1, 64, 0, B, rj) == 0);
        CHECK(oracle_sample_rejection(lg, dt, B, V, STRIDE, T, P, MP, 9, seeds, 1, 1, 0, B, rj) == 0);
        float* q = (float*)malloc(sizeof(float) * B * V);
        int32_t d[B];
        for (int b = 0; b < B; ++b) {
            double s = 0.0;
            for (int i = 0; i < V; ++i) {
                const float w = (b % 3 == 0 && i > 10) ? 0.0f : (float)uniform01();
                q[b * V + i] = w;
                s += w;
            }
            for (int i = 0; i < V; ++i) q[b * V + i] = (float)(q[b * V + i] / s);
            d[b] = b == 23 ? V + 3 : (b == 22 ? -1 : (int32_t)(next_u64() % 12));
        }
        oracle_spec_row sp[B];
        CHECK(oracle_spec_verify(lg, dt, B, V, STRIDE, T, P, K, MP, q, d, 11, NULL, 2, 1e-6, 0, B, sp) == 0);
        CHECK(oracle_spec_verify(lg, dt, B, V, STRIDE, T, P, K, MP, q, d, 11, seeds, 2, 1e-6, 0, B, sp) == 0);
        free(q);
        /* The pre-chain. */
        int32_t hist[B * H];
        float rep[B], fr[B], pres[B];
        uint32_t allowed[B * ((V + 31) / 32)];
        for (int b = 0; b < B; ++b) {
            for (int h = 0; h < H; ++h) {
                const int r = (int)(next_u64() % 16);
                hist[b * H + h] = r == 0 ? -1 : (r == 1 ? V + 9 : (r == 2 ? -7 : (int32_t)(next_u64() % V)));
            }
            rep[b] = (float)(0.5 + uniform01());
            fr[b] = (float)(uniform01() - 0.5);
            pres[b] = (float)uniform01();
            for (int j = 0; j < (V + 31) / 32; ++j) allowed[b * ((V + 31) / 32) + j] = (uint32_t)next_u64();
        }
        float* xo = (float*)malloc(sizeof(float) * B * V);
        CHECK(oracle_preprocess(lg, dt, B, V, STRIDE, hist, H, rep, fr, pres, allowed, xo) == 0);
        CHECK(oracle_preprocess(lg, dt, B, V, STRIDE, NULL, 0, NULL, NULL, NULL, NULL, xo) == 0);
        free(xo);
    }
    /* The level rule, Philox and the noise words. */
    double ord[6] = {0.4, 0.3, 0.3, 0.2, 0.0, 0.0}, mass[6] = {0.4, 0.3, 0.3, 0.2, 0.0, 0.0};
    uint8_t keep[6];
    double a, m;
    CHECK(oracle_topp_levels(ord, mass, 6, 0.5, keep, &a, &m) == 3);
    CHECK(oracle_topp_levels(ord, mass, 6, 1.0, keep, &a, &m) == 6);
    const uint32_t c[4] = {1, 2, 3, 4}, k[2] = {5, 6};
    uint32_t o[4];
    oracle_philox4x32_10(c, k, o);
    uint32_t words[1027];
    oracle_noise_words(1, 2, 3, 1027, words);
    CHECK(words[1026] == oracle_noise_word(1, 2, 3, 1026));
    CHECK(oracle_exp1(0u) > 0.0 && oracle_exp1(0xFFFFFFFFu) > 0.0);
    /* Bad arguments are refused before any access. */
    CHECK(oracle_sample_ex(x, 7, B, V, STRIDE, T, P, K, MP, 0, NULL, 0, 0, B, rows, NULL, NULL) == -1);
    CHECK(oracle_sample_ex(x, 0, B, V, V - 1, T, P, K, MP, 0, NULL, 0, 0, B, rows, NULL, NULL) == -1);
    CHECK(oracle_sample_ex(x, 0, B, V, STRIDE, T, P, K, MP, 0, NULL, 0, 0, B + 1, rows, NULL, NULL) == -1);
    CHECK(oracle_sample_ex(x, 0, B, 0, STRIDE, T, P, K, MP, 0, NULL, 0, 0, B, rows, NULL, NULL) == -1);

#ifdef PLANT_OVERRUN
    /* A read one element past the logits: proves the sanitizer is live. */
    volatile float past = x[B * STRIDE];
    (void)past;
#endif
    free(x);
    free(xb);
    free(probs);
    free(lps);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
