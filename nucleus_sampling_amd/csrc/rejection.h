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

constexpr float kChainDelta = 0.015625f;  // round 1 keeps every score >= 1/64 of the best
constexpr int kChainCap = 512;              // kept scores per wave
constexpr int kChainMax = 4;                // proposals tested by one pass

struct RejShared {
    union {
        RaceQueue rq[kRowThreads / kWave];             // race passes
        u32x2v list[kRowThreads / kWave][kChainCap];   // round 1's high scores: (score bits, index)
    } u;
    ResolveShared rs;
    float redf[kMaxWaves];
    int redi[kMaxWaves];
    double redd[kMaxWaves];
    uint32_t wn[kMaxWaves];  // high scores kept per wave; 0xFFFFFFFF if some were lost
    uint32_t sstar_bits;     // best exact race score so far in the workgroup
};

// Drops the wave's kept scores below thr (all lanes; n the same in every
// lane).  Survivors keep their order.
__device__ __forceinline__ void chain_compact(u32x2v* seg, uint32_t& n, float thr, uint32_t lane)
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint32_t m = 0;
    for (uint32_t base = 0; base < n; base += kWave) {
        const uint32_t i = base + lane;
        const u32x2v e = i < n ? seg[i] : u32x2v{0u, 0u};
        const bool keep = i < n && __uint_as_float(e.x) >= thr;
        const uint64_t mask = __ballot(keep);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (keep) seg[m + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u))] = e;
        m += (uint32_t)__popcll(mask);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    n = m;
}

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
    RaceQueue& rq = sh.u.rq[t / kWave];
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
    // Every token scoring at least 1/64 of the best score so far is kept in
    // its wave's list (the list drops entries that fall below 1/64 of the
    // rising best when it fills), so at the end it holds every token scoring
    // at least 1/64 of the final best: the next proposals, below.
    float lmax = -INFINITY;
    int bad = 0;
    bool racing = false;  // uniform
    RowModel ref = {};
    float c1 = 0.0f;
    RaceAcc acc;
    acc.init();
    float sstar = 0.0f;
    u32x2v* const seg = sh.u.list[t / kWave];
    uint32_t wn = 0;     // the wave's kept scores, as last read (the same in every lane)
    bool lost = false;   // the wave ran out of room for scores it must keep (uniform in the wave)
    if (t == 0) sh.sstar_bits = 0;
    if (lane == 0) sh.wn[t / kWave] = 0;  // (published to the wave by the first hook's barriers)
    stream_row<DT, false, kRowThreads>(
        p, rowp,
        [&](uint32_t i0, const float* xs) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bad |= !(xs[j] < INFINITY);  // NaN or +inf
                lmax = fmaxf(lmax, xs[j]);
            }
            if (!racing) return;  // uniform
            // Screen against 1/64 of the best score any wave has reached: a
            // token is scored exactly unless it provably scores below that
            // (the sampler's log2 screen, race_groups, with the bound scaled).
            const float shared = __uint_as_float(sh.sstar_bits);
            const float bnd = fmaxf(sstar, shared);
            const float thr = kChainDelta * bnd;  // exact: a power of two
            const float q = thr > 0.0f ? -__builtin_amdgcn_logf(thr) + 2e-3f : INFINITY;  // R errs high: see race_groups
            const uint4 w4 = philox4x32_10(make_uint4(i0 >> 2, (uint32_t)b, p.step_lo, p.step_hi), p.seed_lo, p.seed_hi);
            uint32_t pass = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = xs[j];
                const bool fin = x >= -FLT_MAX && x <= FLT_MAX;
                // race_groups' screen in log2 units, against thr.
                const float R = fmaf(x - ref.m, c1, q);
                const float nf = (float)(~philox_word(w4, (uint32_t)j));
                const float L = fmaf((float)__float_as_uint(nf), 0x1p-23f, -159.00005f);
                pass |= (fin && !(L > R)) ? (1u << j) : 0u;
            }
            // Room for this call's appends (at most 4 per lane), compacting
            // the list first if needed (uniform in the wave).
            if (!lost) {
                wn = sh.wn[t / kWave];
                if (wn > (uint32_t)kChainCap - 4 * kWave) {
                    chain_compact(seg, wn, thr, lane);
                    if (lane == 0) sh.wn[t / kWave] = wn;
                    lost = wn > (uint32_t)kChainCap - 4 * kWave;
                }
            }
            while (pass) {
                const uint32_t j = (uint32_t)__builtin_ctz(pass);
                pass &= pass - 1u;
                float x = xs[0];
                x = j == 1 ? xs[1] : x;
                x = j == 2 ? xs[2] : x;
                x = j == 3 ? xs[3] : x;
                const float sc = exact_score(x, ref.m, ref.T, ref.invT, philox_word(w4, j));
                const uint64_t pk = race_pack(sc, i0 + j);
                acc.best = pk > acc.best ? pk : acc.best;
                sstar = fmaxf(sstar, sc);
                if (sc >= thr && !lost) {
                    const uint32_t off = atomicAdd(&sh.wn[t / kWave], 1u);
                    if (off < (uint32_t)kChainCap) {
                        u32x2v e;
                        e.x = __float_as_uint(sc);
                        e.y = i0 + j;
                        seg[off] = e;
                    }
                }
            }
            if (__ballot(sstar > shared)) {
                const float wave_best = wave_reduce(sstar, MaxF());
                if (lane == 0) atomicMax(&sh.sstar_bits, __float_as_uint(wave_best));
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
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (lane == 0 && lost) sh.wn[t / kWave] = 0xFFFFFFFFu;
    block_extremes<kRowThreads>(lmax, bad, sh.redf, sh.redi);  // (its barriers publish wn)
    const float m = uniform(lmax);
    uint64_t best = racing ? block_race<kRowThreads>(acc, sh.rs).best : 0;
    bool chain_ok = racing;
#pragma unroll
    for (int w = 0; w < kRowThreads / kWave; ++w) chain_ok &= sh.wn[w] != 0xFFFFFFFFu;
    chain_ok = uniform((uint32_t)chain_ok) != 0;

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
        if (!racing || (double)(m - ref.m) * (double)ref.invT > 64.0) {
            best = race_pass(true, -FLT_MAX, model);
            chain_ok = false;
        }
        const float cw = model.invT * 1.4426950408889634f;
        auto accepts = [&](float xt, double a, double S) {
            return survives(model, xt) && (xt == m || rp.P >= 1.0f || (rp.P > 0.0f && a < (double)rp.P * S));
        };
        double S = 0.0;
        bool have_S = false;
        int r0 = 1;
        bool done = false;
        if (chain_ok) {
            // ---- the next proposals without racing again.  Round k + 1
            // proposes the best score among tokens above round k's logit; if
            // any token kept above that logit scores >= 1/64 of the best, the
            // best of them is that proposal (every token scoring that much was
            // kept).  Up to four proposals, then one pass tests them all.
            const float s1 = __uint_as_float((uint32_t)(best >> 32));
            const float thr1 = kChainDelta * s1;
            uint32_t tok[kChainMax];
            float xk[kChainMax];
            int K = 1;
            tok[0] = uniform((uint32_t)~(uint32_t)best);
            xk[0] = uniform(logit_at<DT>(rowp, tok[0]));
            const uint32_t wv = (uint32_t)t / kWave;
            const uint32_t nw = sh.wn[wv];
#pragma unroll
            for (int k = 1; k < kChainMax; ++k) {
                uint64_t g = 0;
                for (uint32_t i = lane; i < nw; i += kWave) {
                    const u32x2v e = sh.u.list[wv][i];
                    const float sc = __uint_as_float(e.x);
                    if (sc >= thr1 && logit_at<DT>(rowp, e.y) > xk[K - 1]) {
                        const uint64_t pk = race_pack(sc, e.y);
                        g = pk > g ? pk : g;
                    }
                }
                g = uniform(block_reduce<kRowThreads>(g, MaxU64(), sh.rs.red64));
                if (g == 0 || K < k) break;  // no kept token above: the list cannot tell
                tok[K] = (uint32_t)~(uint32_t)g;
                xk[K] = uniform(logit_at<DT>(rowp, tok[K]));
                ++K;
            }
            float xs4[kChainMax];
#pragma unroll
            for (int k = 0; k < kChainMax; ++k) xs4[k] = k < K ? xk[k] : INFINITY;
            double a[kChainMax] = {0.0, 0.0, 0.0, 0.0}, s = 0.0;
            stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t, const float* xs) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float v = xs[j];
                    const float e = __builtin_amdgcn_exp2f((v - model.m) * cw);
                    const double w = survives(model, v) ? (double)e : 0.0;
                    s += w;
#pragma unroll
                    for (int k = 0; k < kChainMax; ++k) a[k] += v > xs4[k] ? w : 0.0;
                }
            });
            S = block_reduce<kRowThreads>(s, SumF64(), sh.redd);
            have_S = true;
#pragma unroll
            for (int k = 0; k < kChainMax; ++k) a[k] = block_reduce<kRowThreads>(a[k], SumF64(), sh.redd);
            for (int k = 0; k < K && !done; ++k)
                if (accepts(xk[k], a[k], S)) {
                    token = (int32_t)tok[k];
                    rounds = k + 1;
                    done = true;
                }
            if (!done) {
                r0 = K + 1;
                best = race_pass(true, next_up(xk[K - 1]), model);
            }
        }
        for (int r = r0; !done; ++r) {
            const uint32_t tk = uniform((uint32_t)~(uint32_t)best);
            if (tk >= (uint32_t)p.V) break;  // no proposal (cannot happen: the max is above every pivot)
            const float xt = uniform(logit_at<DT>(rowp, tk));
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
            if (!have_S) {
                S = block_reduce<kRowThreads>(s, SumF64(), sh.redd);
                have_S = true;
            }
            if (accepts(xt, a, S)) {
                token = (int32_t)tk;
                rounds = r;
                break;
            }
            if (r >= kMaxRounds) {
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
