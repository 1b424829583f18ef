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

constexpr int kThreads = 256;     // split-row workgroups
constexpr int kMaxWaves = 16;     // largest workgroup: 1024 threads
constexpr int kDigitBins = 256;

struct SelectShared {
    uint64_t hist[kDigitBins];
    uint64_t res_before, res_at, res_total;
    int res_j;
};

struct SelectResult {
    uint32_t level;     // the cut key level L
    uint64_t above;     // total weight of eligible keys > L
    uint64_t at;        // total weight of eligible keys == L
    uint64_t total;     // total eligible weight
};

__device__ __forceinline__ uint64_t lane_read64(uint64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// `visit(fn)` calls fn(key, weight) for every eligible token this thread
// owns (weight > 0; zero-weight tokens are skipped).  Every thread of the
// workgroup (NT >= 64 threads) must call select_level.  `thr_of_total(total)`
// maps the total eligible weight to the threshold.  If no level qualifies
// (thr == 0), the top level is returned; with no eligible token, 0xFFFFFFFF.
//
// Every eligible key lies in [lo_key, hi_key].  The leading digits those two
// share are then every eligible key's digits, and the search above would
// pick exactly them with the weight above unchanged, so they take no pass:
// a crossing bin's tokens usually differ only in their low two digits.
//
// Per digit: all threads add their tokens into the 256-bin LDS histogram;
// then the first wave alone scans it (lane l holds digits 255-4l .. 252-4l,
// highest first), publishes the chosen digit and clears the histogram for
// the next digit.  Two workgroup barriers per digit.
template <int NT, class Visit, class ThrFn>
__device__ __forceinline__ SelectResult select_level(Visit visit, ThrFn thr_of_total, SelectShared& sh,
                                                     uint32_t lo_key = 0u, uint32_t hi_key = 0xFFFFFFFFu)
{
    const uint32_t diff = lo_key ^ hi_key;
    const int first = diff ? min(__builtin_clz(diff) >> 3, 3) : 3;  // at least one pass: it finds the total
    uint32_t mask = first ? 0xFFFFFFFFu << (32 - 8 * first) : 0u;
    uint32_t prefix = lo_key & mask;
    uint64_t base = 0, thr = 0, total = 0;
    const int t = threadIdx.x;
    for (int i = t; i < kDigitBins; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int lvl = first; lvl < 4; ++lvl) {
        const int shift = 24 - 8 * lvl;
        // Each thread sums a run of tokens with one digit in registers and
        // adds it to the histogram when the digit changes; the last runs of
        // a wave go in with one atomic when they share a digit.  Tied keys
        // (a whole level in the crossing bin) would otherwise send every
        // token's atomic to one LDS address.
        uint32_t rd = 0;
        uint64_t racc = 0;
        visit([&](uint32_t key, uint64_t w) {
            if ((key & mask) == prefix) {
                const uint32_t d = (key >> shift) & 0xFFu;
                if (d != rd && racc) {
                    atomicAdd((unsigned long long*)&sh.hist[rd], (unsigned long long)racc);
                    racc = 0;
                }
                rd = d;
                racc += w;
            }
        });
        {
            const bool has = racc != 0;
            const uint64_t hm = __ballot(has);
            if (hm) {  // uniform
                const int leader = (int)__builtin_ctzll(hm);
                const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)rd, leader);
                if (__ballot(has && rd != dl) == 0) {  // uniform: one digit for the whole wave
                    const uint64_t tot = wave_reduce(racc, SumU64());
                    if ((int)(t & (kWave - 1)) == leader)
                        atomicAdd((unsigned long long*)&sh.hist[dl], (unsigned long long)tot);
                } else if (has) {
                    atomicAdd((unsigned long long*)&sh.hist[rd], (unsigned long long)racc);
                }
            }
        }
        __syncthreads();
        if (t < kWave) {
            uint64_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = sh.hist[kDigitBins - 1 - (4 * t + i)];
            const uint64_t ls = h[0] + h[1] + h[2] + h[3];
            // Inclusive prefix of the lane sums; minus the lane's own sum, the
            // weight of the digits above this lane's.
            uint64_t all;
            const uint64_t x = wave_inclusive_sum(ls, all);
            if (lvl == first) {
                total = all;
                thr = thr_of_total(total);
            }
            uint64_t bf = base + x - ls;
            // Lowest non-empty digit whose weight above is < thr (largest rank);
            // failing that, the highest non-empty digit (smallest rank).
            int cand = -1, top = kDigitBins;
            uint64_t cb = 0, ch = 0, tb = 0, th = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rank = 4 * t + i;
                if (h[i] > 0 && bf < thr) {
                    cand = rank;
                    cb = bf;
                    ch = h[i];
                }
                if (h[i] > 0 && rank < top) {
                    top = rank;
                    tb = bf;
                    th = h[i];
                }
                bf += h[i];
            }
            int j = wave_reduce(cand, MaxI32());
            uint64_t jb = base, jh = 0;
            if (j >= 0) {
                jb = lane_read64(cb, j >> 2);
                jh = lane_read64(ch, j >> 2);
            } else {
                j = wave_reduce(top, MinI32());
                if (j < kDigitBins) {
                    jb = lane_read64(tb, j >> 2);
                    jh = lane_read64(th, j >> 2);
                } else {
                    j = 0;  // nothing eligible: level 0xFF.. of the prefix, weight 0
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sh.hist[4 * t + i] = 0;
            if (t == 0) {
                sh.res_j = j;
                sh.res_before = jb;
                sh.res_at = jh;
                if (lvl == first) sh.res_total = total;
            }
        }
        __syncthreads();
        const int j = sh.res_j;
        base = sh.res_before;
        prefix |= (uint32_t)(kDigitBins - 1 - j) << shift;
        mask |= 0xFFu << shift;
    }
    SelectResult r;
    r.total = sh.res_total;
    r.level = r.total ? prefix : 0xFFFFFFFFu;  // (as every digit of an empty search is 0xFF)
    r.above = base;
    r.at = sh.res_at;
    return r;
}

}  // namespace nucleus
