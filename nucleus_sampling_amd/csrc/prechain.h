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
// copy of the row.  Per row, the workgroup stages in LDS a hash table of the
// history and a bit per token: each distinct id with its count and its own
// mask bit goes into one of 512 buckets of four packed words (a full bucket
// spills into the next), every thread inserting its own history entry;
// the staged bits are the mask (all set without one) with every history id
// cleared.  A token whose bit is set is passed as it is, after one 4-byte LDS
// read per four tokens.  A token whose bit is clear is forbidden unless an
// 8K-bit filter of hashed history ids says it may be in the history; then it
// probes the table (one 16-byte read, rarely two): found, it is penalised and
// its own mask bit applied; not found, it is forbidden.
#pragma once

#include "common.h"
#include "params.h"

namespace nucleus {

constexpr int kHistMax = 1024;        // history entries per row
constexpr int kHistBuckets = 512;     // hash buckets of 4 entries: load <= 1/2
constexpr int kFilterWords = 256;     // 8192 filter bits
constexpr int kMaskWordsMax = 5216;   // mask words staged per row: V <= 166912

struct PreShared {
    uint4 table[kHistBuckets];             // entries (allowed << 31) | ((id + 1) << 11) | count, 0 = empty
    uint32_t filter[kFilterWords];         // history ids hashed
    uint32_t mask[kMaskWordsMax];          // pass bits: allowed and not in the history
};

struct PreRow {
    float rho, af, ap;
    bool pen;   // penalties change something on this row (uniform)
    bool mask;  // the row has a mask (uniform)
    uint32_t V;
};

__device__ __forceinline__ uint32_t pre_bucket(uint32_t i) { return (i * 0x9E3779B1u) >> 23; }
__device__ __forceinline__ uint32_t pre_filter_bit(uint32_t i) { return (i * 0x85EBCA77u) >> 19; }

// Stages row b's history table and mask in LDS.  All NT threads (one
// history entry each); ends with a barrier.
//
// Each thread inserts its own history id: it walks the slots from the id's
// bucket on, claims the first empty one by compare-and-swap, or, meeting a
// slot that already holds the id, adds one to that entry's count.  Slots are
// never emptied, so every slot between an id's bucket and its entry is full
// whatever order the threads ran in, which is what the lookup relies on; the
// counts are sums, so the table's contents do not depend on that order.
template <int NT>
__device__ __forceinline__ PreRow pre_setup(const Params& p, int64_t b, PreShared& ps)
{
    static_assert(NT == kHistMax, "one history entry per thread");
    const uint32_t t = threadIdx.x;
    PreRow r;
    r.V = (uint32_t)p.V;
    r.rho = uniform(p.rep_pen ? p.rep_pen[b] : 1.0f);
    r.af = uniform(p.freq_pen ? p.freq_pen[b] : 0.0f);
    r.ap = uniform(p.pres_pen ? p.pres_pen[b] : 0.0f);
    const uint32_t H = (uint32_t)p.hist_len;
    r.pen = p.hist && H > 0 && !(r.rho == 1.0f && r.af == 0.0f && r.ap == 0.0f);
    r.mask = p.allowed != nullptr;
    uint32_t v = 0xFFFFFFFFu;
    if (r.pen && t < H) {
        const int32_t tok = p.hist[b * (int64_t)H + t];
        if (tok >= 0 && (uint32_t)tok < r.V) v = (uint32_t)tok;
    }
    for (uint32_t i = t; i < (uint32_t)kHistBuckets; i += NT) ps.table[i] = make_uint4(0, 0, 0, 0);
    for (uint32_t i = t; i < (uint32_t)kFilterWords; i += NT) ps.filter[i] = 0;
    const uint32_t W = (r.V + 31) >> 5;
    for (uint32_t i = t; i < W; i += NT) ps.mask[i] = r.mask ? p.allowed[b * (int64_t)W + i] : 0xFFFFFFFFu;
    __syncthreads();
    if (v != 0xFFFFFFFFu) {
        const uint32_t allowed = r.mask ? (p.allowed[b * (int64_t)W + (v >> 5)] >> (v & 31)) & 1u : 1u;
        const uint32_t key = (v + 1u) << 11;
        const uint32_t e = (allowed << 31) | key | 1u;
        atomicAnd(&ps.mask[v >> 5], ~(1u << (v & 31)));  // history ids take the slow path
        const uint32_t h = pre_filter_bit(v);
        atomicOr(&ps.filter[h >> 5], 1u << (h & 31));
        uint32_t* slots = (uint32_t*)ps.table;
        const uint32_t s0 = pre_bucket(v) * 4;
        // At most 1024 ids in 2048 slots: an empty or matching slot is met.
        for (uint32_t k = 0; k < 4u * kHistBuckets; ++k) {
            const uint32_t sl = (s0 + k) & (4u * kHistBuckets - 1);
            const uint32_t old = atomicCAS(&slots[sl], 0u, e);
            if (old == 0u) break;
            if ((old & 0x7FFFF800u) == key) {  // the id's entry: count one more
                atomicAdd(&slots[sl], 1u);
                break;
            }
        }
    }
    __syncthreads();
    return r;
}

// Token i's table entry: (allowed << 31) | ((i + 1) << 11) | count, or 0 if
// i is not in the row's history.
__device__ __forceinline__ uint32_t pre_entry(const PreShared& ps, uint32_t i)
{
    const uint32_t key = i + 1u;
    uint32_t bk = pre_bucket(i);
    for (int k = 0; k < kHistBuckets; ++k) {
        const uint4 e = ps.table[bk];
        uint32_t f = 0;
        f = ((e.x >> 11) & 0xFFFFFu) == key ? e.x : f;
        f = ((e.y >> 11) & 0xFFFFFu) == key ? e.y : f;
        f = ((e.z >> 11) & 0xFFFFFu) == key ? e.z : f;
        f = ((e.w >> 11) & 0xFFFFFu) == key ? e.w : f;
        // Found, or the bucket has room (an insertion would have stopped here).
        if (f || e.x == 0 || e.y == 0 || e.z == 0 || e.w == 0) return f;
        bk = (bk + 1) & (kHistBuckets - 1);
    }
    return 0;
}

// Applies the pre-chain to tokens i0 .. i0 + 3 (i0 a multiple of 4; values at
// or past V are -inf already and stay so).  A group with a staged bit clear
// reads its four filter words together, with no branch between them, so it
// waits for LDS once; only tokens the filter cannot clear take the table
// probe.
__device__ __forceinline__ void pre_apply(const PreRow& r, const PreShared& ps, uint32_t i0, float* x)
{
#pragma clang fp contract(off)
    if (i0 >= r.V) return;
    const uint32_t bits = ps.mask[i0 >> 5] >> (i0 & 31);
    if ((bits & 0xFu) == 0xFu) return;  // all four allowed and not in the history
    uint32_t slow = 0;  // bit j: token i0 + j may be in the history
    if (r.pen) {        // uniform
        uint32_t f[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t h = pre_filter_bit(i0 + (uint32_t)j);
            f[j] = ps.filter[h >> 5] >> (h & 31);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) slow |= (f[j] & ~(bits >> j) & 1u) << j;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // A staged bit set: unchanged.  Clear, and not possibly in the
        // history: forbidden.
        const bool pass = (bits >> j) & 1u;
        const bool maybe = (slow >> j) & 1u;
        x[j] = pass || maybe ? x[j] : -INFINITY;
    }
    if (!slow) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (!((slow >> j) & 1u)) continue;
        const uint32_t e = pre_entry(ps, i0 + (uint32_t)j);
        if (e) {
            const uint32_t c = e & 2047u;
            const float y = x[j] > 0.0f ? __fdiv_rn(x[j], r.rho) : x[j] * r.rho;
            float pen = r.af * (float)c;
            pen = pen + r.ap;
            x[j] = (e >> 31) ? y - pen : -INFINITY;
        } else {
            x[j] = -INFINITY;  // forbidden
        }
    }
}

}  // namespace nucleus
