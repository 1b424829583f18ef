// rejection.h -- sort-free top-p by rejection ("Top-p (Nucleus) Sampling, in
// depth", "Sort-free top-p by rejection sampling"): a second way to draw from
// the kept distribution, with no histogram, no cut and no sort.
//
// Per row, with m the row max, e_i = exp((x_i - m)/T), the min-p survivors
// and S their total weight: a pivot starts below every logit.  Each round
// proposes the race winner t = argmax e_i / E_i over the finite tokens above
// the pivot (the same Philox words E_i as the main sampler) and accepts it iff
// it survives min-p and either it is in the top level, or p >= 1, or p > 0
// and the survivor mass strictly above it, A(t), is below p S (the order-free
// rule: ties share a fate, the top level is always kept, p >= 1 keeps every
// survivor).  A rejected t and every token at or below it are out of the
// nucleus: the pivot moves to x_t.
//
// Reusing the words in every round is a valid draw: in arrival-time form the
// race winner is the first token to arrive, and given that the first arrivals
// were rejected, the others' remaining waiting times are again independent
// exponentials with the same rates, so each round proposes in proportion to
// e among the tokens above the pivot.  The accepted token is then the first
// kept token to arrive: the main sampler's token, reached without finding the
// cut.
//
// One 1024-thread workgroup per row.  The first round's race runs in the pass
// that finds the max, against the max of the first tokens loaded (scores
// relative to any common reference pick the same winner); each acceptance
// test is one pass summing survivor weights (the first one also S), and each
// further round one race pass over the tokens above the pivot.  A row that
// accepts in round r streams the row 2r times.  Sums are in double, each
// thread in a fixed order and the workgroup in a fixed order: deterministic.
// Weights in the test come from exp2 of the scaled logit difference, within
// about |x - m|/T * 1e-7 relative of e (1e-6 below e = 1e-9, where tokens no
// longer move S).
#pragma once

#include <float.h>

#include "rowpath.h"

namespace nucleus {

constexpr int kMaxRounds = 64;  // a row needs at most one round per distinct logit

struct SumF64 {
    __device__ double operator()(double a, double b) const { return a + b; }
};

struct RejShared {
    RaceQueue rq[kRowThreads / kWave];
    ResolveShared rs;
    float redf[kMaxWaves];
    int redi[kMaxWaves];
    double redd[kMaxWaves];
    uint32_t sstar_bits;  // best exact race score so far in the workgroup
};

template <int DT>
__device__ __forceinline__ float logit_at(const void* rowp, uint32_t i)
{
    return DT == kF32 ? ((const float*)rowp)[i] : bf16_to_float(((const uint16_t*)rowp)[i]);
}

// The smallest float strictly above x (x finite).
__device__ __forceinline__ float next_up(float x) { return key_value(order_key(x) + 1u); }

template <int DT>
__global__ __launch_bounds__(kRowThreads, 1) void rejection_kernel(Params p, int32_t* out_rounds)
{
    __shared__ RejShared sh;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    use_row_key(p, b);
    const RowParams rp = row_params(p, b);
    const uint32_t lane = (uint32_t)t & (kWave - 1);
    RaceQueue& rq = sh.rq[t / kWave];
    const bool tempered = rp.T > 0.0f;  // false for T <= 0 and NaN

    // One race over the tokens with x >= lo (scored: e/E against the
    // reference ref.m; unscored: the lowest index), as a pass of its own.
    auto race_pass = [&](bool scored, float lo, const RowModel& ref) -> uint64_t {
        __syncthreads();  // the queues and the shared bound are free
        if (t == 0) sh.sstar_bits = 0;
        __syncthreads();
        RaceAcc a;
        a.init();
        float ss = 0.0f;
        uint32_t qh = 0, qn = 0;
        const float cl = ref.invT * 1.4426950408889634f;
        auto race = [&](const uint32_t* i0, const float (*xs)[4], const bool* active) __attribute__((always_inline)) {
            race_queued(p, b, scored, ref, cl, lo, i0, xs, active, a, ss, &sh.sstar_bits, false);
        };
        stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
            const bool any = (xs[0] >= lo) | (xs[1] >= lo) | (xs[2] >= lo) | (xs[3] >= lo);
            wq_push(rq, qh, qn, lane, any, i0, xs, race);
        });
        if (qn) wq_drain(rq, qh, qn, lane, qn, race);
        return block_race<kRowThreads>(a, sh.rs).best;
    };

    // ---- round 1's race, fused with the row max and the NaN / +inf check:
    // every finite token races against the max of the first tokens loaded.
    float lmax = -INFINITY;
    int bad = 0;
    bool racing = false;  // uniform
    RowModel ref = {};
    float c1 = 0.0f;
    RaceAcc acc;
    acc.init();
    float sstar = 0.0f;
    uint32_t qh = 0, qn = 0;
    if (t == 0) sh.sstar_bits = 0;
    auto race1 = [&](const uint32_t* i0, const float (*xs)[4], const bool* active) __attribute__((always_inline)) {
        race_queued(p, b, true, ref, c1, -FLT_MAX, i0, xs, active, acc, sstar, &sh.sstar_bits, false);
    };
    stream_row<DT, false, kRowThreads>(
        p, rowp,
        [&](uint32_t i0, const float* xs) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bad |= !(xs[j] < INFINITY);  // NaN or +inf
                lmax = fmaxf(lmax, xs[j]);
            }
            if (racing) {
                const bool any = (xs[0] >= -FLT_MAX) | (xs[1] >= -FLT_MAX) | (xs[2] >= -FLT_MAX) | (xs[3] >= -FLT_MAX);
                wq_push(rq, qh, qn, lane, any, i0, xs, race1);
            }
        },
        [&](float mx) {
            if (!tempered) return;
            const float m1 = block_reduce<kRowThreads>(mx, MaxF(), sh.redf);
            racing = m1 > -INFINITY && m1 < INFINITY;
            if (racing) {
                ref = uniform(make_model(m1, rp.T, 0.0f));
                c1 = ref.invT * 1.4426950408889634f;
            }
        });
    if (racing && qn) wq_drain(rq, qh, qn, lane, qn, race1);
    block_extremes<kRowThreads>(lmax, bad, sh.redf, sh.redi);
    const float m = uniform(lmax);
    uint64_t best = racing ? block_race<kRowThreads>(acc, sh.rs).best : 0;

    int32_t token = -1, rounds = 0;
    if (bad || rp.T != rp.T || rp.P != rp.P || rp.MP != rp.MP || !(m > -INFINITY)) {
        // row error
    } else if (!tempered) {  // greedy: the lowest index among the maximal logits
        RowModel none = {};
        token = (int32_t)~(uint32_t)race_pass(false, m, none);
    } else {
        const RowModel model = uniform(make_model(m, rp.T, rp.MP));
        // Scores against the first tokens' max stay finite while the true max
        // is at most 64 T above it (e <= e^64, E >= 2^-34); otherwise race again
        // against the true max.
        if (!racing || (double)(m - ref.m) * (double)ref.invT > 64.0) best = race_pass(true, -FLT_MAX, model);
        const float cw = model.invT * 1.4426950408889634f;
        double S = 0.0;
        for (int r = 1;; ++r) {
            const uint32_t tok = uniform((uint32_t)~(uint32_t)best);
            if (tok >= (uint32_t)p.V) break;  // no proposal (cannot happen: the max is above every pivot)
            const float xt = uniform(logit_at<DT>(rowp, tok));
            // ---- the acceptance test: survivor mass strictly above x_t (and,
            // the first time, the total survivor mass S)
            double a = 0.0, s = 0.0;
            stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t, const float* xs) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v = xs[j];
                    const float e = __builtin_amdgcn_exp2f((v - model.m) * cw);
                    const double w = survives(model, v) ? (double)e : 0.0;
                    s += w;
                    a += v > xt ? w : 0.0;
                }
            });
            a = block_reduce<kRowThreads>(a, SumF64(), sh.redd);
            if (r == 1) S = block_reduce<kRowThreads>(s, SumF64(), sh.redd);
            const bool accept =
                survives(model, xt) && (xt == m || rp.P >= 1.0f || (rp.P > 0.0f && a < (double)rp.P * S));
            if (accept) {
                token = (int32_t)tok;
                rounds = r;
                break;
            }
            if (r == kMaxRounds) {
                rounds = r;
                break;
            }
            // ---- the next round: race the tokens strictly above x_t
            best = race_pass(true, next_up(xt), model);
        }
    }
    if (t == 0) {
        p.out_token[b] = token;
        if (out_rounds) out_rounds[b] = rounds;
    }
}

}  // namespace nucleus
