// prechain.h -- the steps before the sampler ("Top-p (Nucleus) Sampling, in
// depth", "Where top-p sits in the sampler chain": penalties on the logits,
// then the grammar mask, then temperature and the filters; "What do
// temperature, top-k and top-p ...", "What interviewers probe next":
// penalties act on raw logits so that they change the greedy choice too).
// The pages name the penalties without formulas; the common definitions are
// taken, each step one IEEE float operation in this order (no fused
// multiply-add), so the processed logit is an exact fp32 value:
//
//   c_i = occurrences of token i in the row's history (duplicates count)
//   for c_i > 0:  y = x > 0 ? x / rho : x * rho          (repetition, rho)
//                 x' = y - (a_f * c_i + a_p)              (frequency, presence)
//   x' = -inf where bit (i mod 32) of mask word i / 32 is clear
//
// The row kernel applies this to every register buffer as it arrives, in
// every pass, so the sampler sees only processed logits and never a second
// copy of the row.  Per row, the workgroup stages in LDS the row's mask words
// and a hash table of the history: the ids are sorted (bitonic sort, one per
// thread), each distinct id with its count goes into one of 512 buckets of
// four packed (id + 1, count) words (a full bucket spills into the next), so
// a token's count is one 16-byte LDS read, rarely two.
#pragma once

#include "common.h"
#include "params.h"

namespace nucleus {

constexpr int kHistMax = 1024;        // history entries per row
constexpr int kHistBuckets = 512;     // hash buckets of 4 entries: load <= 1/2
constexpr int kMaskWordsMax = 5472;   // mask words staged per row: V <= 175104

struct PreShared {
    uint4 table[kHistBuckets];             // entries ((id + 1) << 11) | count, 0 = empty
    uint32_t mask[kMaskWordsMax];
};

struct PreRow {
    float rho, af, ap;
    bool pen;   // penalties change something on this row (uniform)
    bool mask;  // the row has a mask (uniform)
    uint32_t V;
};

__device__ __forceinline__ uint32_t pre_bucket(uint32_t i) { return (i * 0x9E3779B1u) >> 23; }

// Stages row b's history table and mask in LDS.  `hs` is kHistMax words of
// LDS free until the call returns (the sort's space).  All NT threads; ends
// with a barrier.
template <int NT>
__device__ __forceinline__ PreRow pre_setup(const Params& p, int64_t b, PreShared& ps, uint32_t* hs)
{
    static_assert(NT == kHistMax, "the bitonic sort takes one history entry per thread");
    const uint32_t t = threadIdx.x;
    PreRow r;
    r.V = (uint32_t)p.V;
    r.rho = uniform(p.rep_pen ? p.rep_pen[b] : 1.0f);
    r.af = uniform(p.freq_pen ? p.freq_pen[b] : 0.0f);
    r.ap = uniform(p.pres_pen ? p.pres_pen[b] : 0.0f);
    const uint32_t H = (uint32_t)p.hist_len;
    r.pen = p.hist && H > 0 && !(r.rho == 1.0f && r.af == 0.0f && r.ap == 0.0f);
    r.mask = p.allowed != nullptr;
    {
        uint32_t v = 0xFFFFFFFFu;
        if (r.pen && t < H) {
            const int32_t tok = p.hist[b * (int64_t)H + t];
            if (tok >= 0 && (uint32_t)tok < r.V) v = (uint32_t)tok;
        }
        hs[t] = v;
    }
    for (uint32_t i = t; i < (uint32_t)kHistBuckets; i += NT) ps.table[i] = make_uint4(0, 0, 0, 0);
    if (r.mask) {
        const uint32_t W = (r.V + 31) >> 5;
        for (uint32_t i = t; i < W; i += NT) ps.mask[i] = p.allowed[b * (int64_t)W + i];
    }
    if (r.pen) {  // uniform
        // Bitonic sort, ascending.
        for (uint32_t k = 2; k <= (uint32_t)kHistMax; k <<= 1)
            for (uint32_t j = k >> 1; j > 0; j >>= 1) {
                __syncthreads();
                const uint32_t o = t ^ j;
                if (o > t) {
                    const uint32_t a = hs[t], c = hs[o];
                    const bool up = (t & k) == 0;
                    if ((a > c) == up) {
                        hs[t] = c;
                        hs[o] = a;
                    }
                }
            }
        __syncthreads();
        // The first thread of each run of equal ids inserts the id with the
        // run's length: a compare-and-swap into the first empty slot from its
        // bucket on (distinct ids only, so no slot is ever counted twice).
        const uint32_t v = hs[t];
        if (v != 0xFFFFFFFFu && (t == 0 || hs[t - 1] != v)) {
            uint32_t n = 1;
            while (t + n < (uint32_t)kHistMax && hs[t + n] == v) ++n;
            const uint32_t e = ((v + 1u) << 11) | n;
            uint32_t* slots = (uint32_t*)ps.table;
            uint32_t s0 = pre_bucket(v) * 4;
            for (uint32_t k = 0; k < 4u * kHistBuckets; ++k) {  // at most 1024 ids in 2048 slots: ends
                const uint32_t s = (s0 + k) & (4u * kHistBuckets - 1);
                if (atomicCAS(&slots[s], 0u, e) == 0u) break;
            }
        }
    }
    __syncthreads();
    return r;
}

// Occurrences of token i in the row's history (0 if none).
__device__ __forceinline__ uint32_t pre_count(const PreShared& ps, uint32_t i)
{
    const uint32_t key = i + 1u;
    uint32_t bk = pre_bucket(i);
    for (int k = 0; k < kHistBuckets; ++k) {
        const uint4 e = ps.table[bk];
        uint32_t c = 0;
        c = (e.x >> 11) == key ? (e.x & 2047u) : c;
        c = (e.y >> 11) == key ? (e.y & 2047u) : c;
        c = (e.z >> 11) == key ? (e.z & 2047u) : c;
        c = (e.w >> 11) == key ? (e.w & 2047u) : c;
        // Found, or the bucket has room (an insertion would have stopped here).
        if (c || e.x == 0 || e.y == 0 || e.z == 0 || e.w == 0) return c;
        bk = (bk + 1) & (kHistBuckets - 1);
    }
    return 0;
}

// Applies the pre-chain to tokens i0 .. i0 + 3 (i0 a multiple of 4; values at
// or past V are -inf already and stay so).
__device__ __forceinline__ void pre_apply(const PreRow& r, const PreShared& ps, uint32_t i0, float* x)
{
#pragma clang fp contract(off)
    if (i0 >= r.V) return;
    if (r.pen) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t c = pre_count(ps, i0 + (uint32_t)j);
            if (c) {
                const float y = x[j] > 0.0f ? __fdiv_rn(x[j], r.rho) : x[j] * r.rho;
                float pen = r.af * (float)c;
                pen = pen + r.ap;
                x[j] = y - pen;
            }
        }
    }
    if (r.mask) {
        const uint32_t bits = ps.mask[i0 >> 5] >> (i0 & 31);
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = ((bits >> j) & 1u) ? x[j] : -INFINITY;
    }
}

}  // namespace nucleus
