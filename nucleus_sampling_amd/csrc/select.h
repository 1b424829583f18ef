// select.h -- exact cut search by radix select over order-preserving keys.
//
// "Find the threshold ... with no sort" ("Implement batched top-p sampling
// with temperature", "What interviewers probe next"): instead of bisecting on
// probability values, the 32-bit key of each eligible token is consumed 8
// bits at a time, most significant first.  A 256-bin LDS histogram of integer
// weights per digit tells which digit holds the answer; four passes give the
// exact key level.  The question answered is always the same:
//
//     the lowest key level L among eligible tokens whose total weight
//     strictly above L is < thr
//
// With weight 1 per token and thr = k it is the top-k cut (ties at the k-th
// value kept); with tempered weights and thr the integer form of p * S it is
// the top-p cut of the order-free rule.  Integer weights make every sum exact,
// so the answer does not depend on the order tokens are visited in.
#pragma once

#include "common.h"

namespace nucleus {

constexpr int kThreads = 256;
constexpr int kDigitBins = 256;

struct SelectShared {
    uint64_t hist[kDigitBins];
    uint64_t red64[kThreads / kWave];
    int redi[kThreads / kWave];
    uint64_t bcast;
};

struct SelectResult {
    uint32_t level;     // the cut key level L
    uint64_t above;     // total weight of eligible keys > L
    uint64_t at;        // total weight of eligible keys == L
    uint64_t total;     // total eligible weight
};

// `visit(fn)` calls fn(key, weight) for every eligible token this thread
// owns (weight > 0; zero-weight tokens are skipped).  Every thread of the
// workgroup must call select_level.  `thr_of_total(total)` maps the total
// eligible weight to the threshold (called once, uniformly).  If no level
// qualifies (thr == 0), the top level is returned.
template <class Visit, class ThrFn>
__device__ SelectResult select_level(Visit visit, ThrFn thr_of_total, SelectShared& sh)
{
    uint32_t prefix = 0, mask = 0;
    uint64_t base = 0, thr = 0, total = 0, at = 0;
    const int t = threadIdx.x;
    for (int lvl = 0; lvl < 4; ++lvl) {
        const int shift = 24 - 8 * lvl;
        sh.hist[t] = 0;
        __syncthreads();
        visit([&](uint32_t key, uint64_t w) {
            if ((key & mask) == prefix)
                atomicAdd((unsigned long long*)&sh.hist[(key >> shift) & 0xFFu], (unsigned long long)w);
        });
        __syncthreads();
        // Thread t owns digit d = 255 - t, so threads run from the top digit down.
        const int d = kDigitBins - 1 - t;
        const uint64_t hw = sh.hist[d];
        if (lvl == 0) {
            total = block_reduce<kThreads>(hw, SumU64(), sh.red64);
            thr = thr_of_total(total);
        }
        const uint64_t before = base + block_exclusive_sum<kThreads>(hw, sh.red64);
        // Lowest non-empty digit whose weight above is < thr; if none (thr == 0),
        // the highest non-empty digit.
        const int cand = (hw > 0 && before < thr) ? t : -1;
        int j = block_reduce<kThreads>(cand, MaxI32(), sh.redi);
        if (j < 0) {
            const int top = (hw > 0) ? (kDigitBins - 1 - t) : -1;  // smallest t with weight
            j = kDigitBins - 1 - block_reduce<kThreads>(top, MaxI32(), sh.redi);
        }
        if (t == j) {
            sh.bcast = before;
            sh.hist[0] = hw;  // safe: every thread has read its own bin above
        }
        __syncthreads();
        base = sh.bcast;
        at = sh.hist[0];
        __syncthreads();
        prefix |= (uint32_t)(kDigitBins - 1 - j) << shift;
        mask |= 0xFFu << shift;
    }
    SelectResult r;
    r.level = prefix;
    r.above = base;
    r.at = at;
    r.total = total;
    return r;
}

}  // namespace nucleus
