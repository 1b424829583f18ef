// row_kernel.h -- one workgroup per row: the general, exact sampler.
//
// Every row is handled by one 1024-thread workgroup that streams the row from
// global memory once per phase:
//
//   1. validate + max: NaN/+inf detection, finite count, the maximal key with
//      its lowest index (a u64 max of key<<32 | ~index);
//   2. min-p: one float threshold on the logit, derived in double from the
//      row max (p_i >= min_p * p_max  <=>  x_i >= max + T ln min_p);
//   3. top-k: a radix select over the 32-bit keys of the survivors, weighting
//      each token 1, for the lowest key level with fewer than k survivors
//      strictly above it (ties at the k-th value survive);
//   4. top-p: the same radix select weighting each survivor by its tempered
//      weight in 2^-40 fixed point, for the lowest level whose mass strictly
//      above is < p * S (the order-free rule; integer sums keep it exact and
//      run-to-run deterministic);
//   5. the exponential race over the kept tokens, the keep count, the kept
//      mass and the smallest kept key; then optionally the renormalised
//      probabilities.
//
// Re-reads come from L2/MALL.  The split-row kernel replaces this on the
// large-vocabulary path; this kernel stays the reference path for every
// shape and the fallback.
#pragma once

#include "common.h"
#include "params.h"

namespace nucleus {

constexpr int kRowBlock = 1024;
constexpr int kRowBins = 2048;

template <int DT>
__device__ __forceinline__ void load_group(const Params& p, const void* rowp, int64_t i0, float x[4])
{
    const int64_t V = p.V;
    if (DT == kF32) {
        const float* r = (const float*)rowp;
        if (p.vec_in && i0 + 4 <= V) {
            const f32x4 v = __builtin_nontemporal_load((const f32x4*)(r + i0));
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = (i0 + j < V) ? r[i0 + j] : -INFINITY;
        }
    } else {
        const uint16_t* r = (const uint16_t*)rowp;
        if (p.vec_in && i0 + 4 <= V) {
            const u32x2 v = __builtin_nontemporal_load((const u32x2*)(r + i0));
            x[0] = __uint_as_float(v.x << 16);
            x[1] = __uint_as_float(v.x & 0xFFFF0000u);
            x[2] = __uint_as_float(v.y << 16);
            x[3] = __uint_as_float(v.y & 0xFFFF0000u);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = (i0 + j < V) ? bf16_to_float(r[i0 + j]) : -INFINITY;
        }
    }
}

// Calls f(group, x[4]) for every 4-token group of the row; tokens past V
// read as -inf (never finite, never kept).
template <int DT, class F>
__device__ __forceinline__ void row_groups(const Params& p, const void* rowp, F&& f)
{
    const int64_t ng = (p.V + 3) >> 2;
    for (int64_t g = threadIdx.x; g < ng; g += kRowBlock) {
        float x[4];
        load_group<DT>(p, rowp, g << 2, x);
        f(g, x);
    }
}

struct RowShared {
    uint64_t hist[kRowBins];
    uint64_t red64[kRowBlock / kWave];
    uint32_t red32[kRowBlock / kWave];
    int redi[kRowBlock / kWave];
    uint64_t bcast64;
    int bcasti;
};

// Lowest non-empty digit whose weight strictly above (base + heavier digits)
// is < thr.  Digits are scanned from the top; returns -1 if none.
template <int NB>
__device__ __forceinline__ int pick_digit(RowShared& sh, uint64_t base, uint64_t thr, uint64_t* before_out)
{
    constexpr int per = NB / kRowBlock;  // 2 for 11-bit digits, 1 for 10-bit
    const int t = threadIdx.x;
    uint64_t local = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) local += sh.hist[NB - 1 - (t * per + q)];
    uint64_t before = base + block_exclusive_sum<kRowBlock>(local, sh.red64);
    int best = -1;
    uint64_t best_before = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        const int d = NB - 1 - (t * per + q);
        const uint64_t w = sh.hist[d];
        if (w > 0 && before < thr) { best = t * per + q; best_before = before; }
        before += w;
    }
    const int j = block_reduce<kRowBlock>(best, MaxI32(), sh.redi);
    if (j >= 0 && best == j) sh.bcast64 = best_before;
    __syncthreads();
    *before_out = (j >= 0) ? sh.bcast64 : 0;
    __syncthreads();
    return (j >= 0) ? NB - 1 - j : -1;
}

// Radix select over 32-bit keys in three digits (11, 11, 10 bits): the lowest
// key level L among eligible tokens with W(keys > L) < thr, where W sums
// weight(x) over eligible tokens.  *above_out receives W(keys > L).
// eligible(x, key) and weight(x) are evaluated per token on each pass.
template <int DT, class Elig, class Wt>
__device__ uint32_t radix_select(const Params& p, const void* rowp, RowShared& sh, uint64_t thr_in,
                                 bool thr_from_total, float ptop, Elig eligible, Wt weight,
                                 uint64_t* above_out, uint64_t* total_out)
{
    uint32_t prefix = 0, mask = 0;
    uint64_t base = 0, thr = thr_in;
    constexpr int shifts[3] = {21, 10, 0};
    constexpr int bits[3] = {11, 11, 10};
#pragma unroll
    for (int lvl = 0; lvl < 3; ++lvl) {
        const int sh_ = shifts[lvl];
        const uint32_t dmask = (1u << bits[lvl]) - 1u;
        for (int i = threadIdx.x; i < kRowBins; i += kRowBlock) sh.hist[i] = 0;
        __syncthreads();
        row_groups<DT>(p, rowp, [&](int64_t g, const float* x) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t k = order_key(x[j]);
                if ((k & mask) == prefix && eligible(x[j], k)) {
                    const uint64_t w = weight(x[j]);
                    if (w) atomicAdd((unsigned long long*)&sh.hist[(k >> sh_) & dmask], (unsigned long long)w);
                }
            }
        });
        __syncthreads();
        if (lvl == 0) {
            uint64_t tot = 0;
            for (int i = threadIdx.x; i < kRowBins; i += kRowBlock) tot += sh.hist[i];
            tot = block_reduce<kRowBlock>(tot, SumU64(), sh.red64);
            *total_out = tot;
            if (thr_from_total) thr = ceil_p_times(ptop, tot);
        }
        uint64_t before;
        const int d = (lvl < 2) ? pick_digit<kRowBins>(sh, base, thr, &before)
                                : pick_digit<kRowBins / 2>(sh, base, thr, &before);
        if (d < 0) {  // nothing qualifies: callers only ask when the top level does
            *above_out = base;
            return prefix;
        }
        base = before;
        prefix |= (uint32_t)d << sh_;
        mask |= dmask << sh_;
    }
    *above_out = base;
    return prefix;
}

template <int DT>
__global__ __launch_bounds__(kRowBlock) void row_sample_kernel(Params p)
{
    __shared__ RowShared sh;
    const int64_t b = blockIdx.x;
    const int64_t esz = (DT == kF32) ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    float* prow = p.out_probs ? p.out_probs + b * p.V : nullptr;

    // 1. validate + max.
    int err = 0;
    uint64_t cnt = 0, best = 0;
    row_groups<DT>(p, rowp, [&](int64_t g, const float* x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = x[j];
            if (v != v || v == INFINITY) err = 1;
            if (v > -INFINITY) {
                ++cnt;
                const uint64_t pk = ((uint64_t)order_key(v) << 32) | (uint64_t)(~(uint32_t)((g << 2) + j));
                best = pk > best ? pk : best;
            }
        }
    });
    err = block_reduce<kRowBlock>(err, OrI32(), sh.redi);
    cnt = block_reduce<kRowBlock>(cnt, SumU64(), sh.red64);
    best = block_reduce<kRowBlock>(best, MaxU64(), sh.red64);

    const float T = p.temperature[b];
    const float P = p.top_p[b];
    const float MP = p.min_p ? p.min_p[b] : 0.0f;
    const int K = p.top_k ? p.top_k[b] : 0;
    if (T != T || P != P || MP != MP || cnt == 0) err = 1;

    if (err) {
        if (threadIdx.x == 0) {
            p.out_token[b] = -1;
            p.out_count[b] = 0;
            if (p.out_min_kept) p.out_min_kept[b] = __uint_as_float(0x7FC00000u);
        }
        if (prow)
            for (int64_t i = threadIdx.x; i < p.V; i += kRowBlock) prow[i] = 0.0f;
        return;
    }
    const uint32_t maxkey = (uint32_t)(best >> 32);
    const uint32_t argmax = ~(uint32_t)best;
    const float m = key_value(maxkey);

    if (T <= 0.0f) {  // greedy
        if (threadIdx.x == 0) {
            p.out_token[b] = (int32_t)argmax;
            p.out_count[b] = 1;
            if (p.out_min_kept) p.out_min_kept[b] = m;
        }
        if (prow)
            for (int64_t i = threadIdx.x; i < p.V; i += kRowBlock) prow[i] = (i == argmax) ? 1.0f : 0.0f;
        return;
    }
    const float invT = (T == INFINITY) ? 0.0f : 1.0f / T;

    // 2. min-p: survivors are x >= t, t = m + T ln(min_p) rounded up to fp32.
    uint32_t cut = 0;  // keep iff finite and key >= cut
    const float mp = MP > 1.0f ? 1.0f : MP;
    if (mp > 0.0f && invT != 0.0f) {
        const double t = (double)m + (double)T * log((double)mp);
        float tf = (float)t;
        if ((double)tf < t) tf = nextafterf(tf, INFINITY);
        if (tf > -INFINITY) cut = order_key(tf);
    }

    // 3. top-k over the min-p survivors.
    if (K > 0) {
        uint64_t above, total;
        const uint32_t c0 = cut;
        const uint32_t kk = radix_select<DT>(
            p, rowp, sh, (uint64_t)K, false, 0.0f,
            [&](float x, uint32_t k) { return x > -INFINITY && k >= c0; },
            [&](float) { return (uint64_t)1; }, &above, &total);
        if (total > (uint64_t)K && kk > cut) cut = kk;
    }

    // 4. top-p over the min-p/top-k survivors, renormalised.
    if (P < 1.0f) {
        if (P <= 0.0f) {
            cut = maxkey;  // only the top level
        } else {
            uint64_t above, total;
            const uint32_t c0 = cut;
            const int shift = p.mass_shift;
            const uint32_t pk = radix_select<DT>(
                p, rowp, sh, 0, true, P,
                [&](float x, uint32_t k) { return x > -INFINITY && k >= c0; },
                [&](float x) { return to_fixed(tempered_weight(x, m, T, invT), shift); }, &above, &total);
            if (pk > cut) cut = pk;
        }
    }

    // 5. race over the kept set, count, kept mass, smallest kept key.
    uint64_t win = 0, kept = 0, mass = 0;
    uint32_t minkey = 0xFFFFFFFFu;
    const int shift = p.mass_shift;
    row_groups<DT>(p, rowp, [&](int64_t g, const float* x) {
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) any |= (x[j] > -INFINITY) && order_key(x[j]) >= cut;
        if (!any) return;
        const uint4 w4 = philox4x32_10(make_uint4((uint32_t)g, (uint32_t)b, p.step_lo, p.step_hi), p.seed_lo,
                                       p.seed_hi);
        const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t k = order_key(x[j]);
            if (!(x[j] > -INFINITY) || k < cut) continue;
            const float e = tempered_weight(x[j], m, T, invT);
            const float s = e / exp1_from_word(words[j]);
            const uint64_t pk = race_pack(s, (uint32_t)((g << 2) + j));
            win = pk > win ? pk : win;
            ++kept;
            mass += to_fixed(e, shift);
            minkey = k < minkey ? k : minkey;
        }
    });
    win = block_reduce<kRowBlock>(win, MaxU64(), sh.red64);
    kept = block_reduce<kRowBlock>(kept, SumU64(), sh.red64);
    mass = block_reduce<kRowBlock>(mass, SumU64(), sh.red64);
    minkey = block_reduce<kRowBlock>(minkey, MinU32(), sh.red32);

    if (threadIdx.x == 0) {
        p.out_token[b] = (int32_t)(~(uint32_t)win);
        p.out_count[b] = (int32_t)kept;
        if (p.out_min_kept) p.out_min_kept[b] = key_value(minkey);
    }
    if (prow) {
        const float inv = (float)(1.0 / ((double)mass * ldexp(1.0, -shift)));
        row_groups<DT>(p, rowp, [&](int64_t g, const float* x) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = (g << 2) + j;
                if (i >= p.V) break;
                const bool keep = (x[j] > -INFINITY) && order_key(x[j]) >= cut;
                prow[i] = keep ? tempered_weight(x[j], m, T, invT) * inv : 0.0f;
            }
        });
    }
}

}  // namespace nucleus
