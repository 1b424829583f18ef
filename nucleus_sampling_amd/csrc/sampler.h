// sampler.h -- the sampler's kernels.
//
// tile_kernel (the fast path, rows up to kMaxChunks * kChunk tokens):
//   each row is split into K chunks of kChunk tokens; one 256-thread
//   workgroup per chunk loads its chunk once from HBM into registers and
//   keeps it there for every phase.  The K workgroups of a row meet at
//   per-row barriers in the workspace; the last to arrive at each barrier
//   merges what the others published and releases them:
//     A  row max, error flag                              -> row mode
//     B  bin histograms of the survivors (model.h)         -> crossing bin
//     C  race partials over the tokens surely kept, and the compacted tokens
//        of the crossing bin -> the last arriver resolves the exact cut
//        (select.h), races the kept candidates and writes the row's outputs.
//   With out_probs the workgroups wait once more and write the renormalised
//   probabilities of their chunk from registers.
//   Workgroups of a row are consecutive in dispatch order on one XCD lane
//   (blockIdx = ((row / 8) * K + chunk) * 8 + row % 8), and dispatch is in
//   order, so the members of the lowest unfinished row are always resident
//   and the barriers cannot deadlock; a bounded spin turns a violation of that
//   assumption into a row error (token -2) instead of a hang.
//
// row_kernel: one 1024-thread workgroup per row (a CU each) streaming the
//   row from global memory once per phase with many loads in flight; the
//   crossing bin's tokens are compacted into LDS for the resolver.  Same
//   decisions, same arithmetic.  It serves batches large enough to fill the
//   device with rows, and rows too long for the split path.
#pragma once

#include <stddef.h>

#include "common.h"
#include "model.h"
#include "params.h"
#include "select.h"
#include "workspace.h"

namespace nucleus {

constexpr int kEPT = 32;                  // tokens per thread held in registers
constexpr int kChunk = kThreads * kEPT;   // tokens per workgroup
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kCandLds = 3072;             // candidates the resolver stages in LDS
constexpr int kMergeBatch = 4;           // loads in flight per thread in the histogram merge

struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct MinF { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct SumU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };

// ---------------------------------------------------------------------------
// Loads: four consecutive tokens starting at i0 (a multiple of 4); tokens at or
// past V read as -inf, which is never finite and never kept.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void load4(const void* rowp, int64_t i0, int64_t V, int vec, float x[4])
{
    if (DT == kF32) {
        const float* r = (const float*)rowp;
        if (vec && i0 + 4 <= V) {
            const f32x4 v = __builtin_nontemporal_load((const f32x4*)(r + i0));
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = (i0 + j < V) ? r[i0 + j] : -INFINITY;
        }
    } else {
        const uint16_t* r = (const uint16_t*)rowp;
        if (vec && i0 + 4 <= V) {
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

// Loads a workgroup's chunk into registers: x[4v + j] is token
// lane0 + 1024 v + j.  Full, aligned chunks take straight-line vector loads
// (the branch is uniform); otherwise every token is loaded from a clamped
// address and masked, without divergent branches.
template <int DT, int EPT>
__device__ __forceinline__ void load_chunk(const void* rowp, uint32_t lane0, uint32_t chunk_end, uint32_t V, int vec,
                                           float x[EPT])
{
    if (vec && chunk_end <= V) {
        if (DT == kF32) {
            const float* r = (const float*)rowp;
#pragma unroll
            for (int v = 0; v < EPT / 4; ++v) {
                const f32x4 q = __builtin_nontemporal_load((const f32x4*)(r + lane0 + (uint32_t)v * (kThreads * 4)));
                x[4 * v] = q.x; x[4 * v + 1] = q.y; x[4 * v + 2] = q.z; x[4 * v + 3] = q.w;
            }
        } else {
            const uint16_t* r = (const uint16_t*)rowp;
#pragma unroll
            for (int v = 0; v < EPT / 4; ++v) {
                const u32x2 q = __builtin_nontemporal_load((const u32x2*)(r + lane0 + (uint32_t)v * (kThreads * 4)));
                x[4 * v] = __uint_as_float(q.x << 16);
                x[4 * v + 1] = __uint_as_float(q.x & 0xFFFF0000u);
                x[4 * v + 2] = __uint_as_float(q.y << 16);
                x[4 * v + 3] = __uint_as_float(q.y & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const uint32_t i = lane0 + (uint32_t)(e >> 2) * (kThreads * 4) + (uint32_t)(e & 3);
            const uint32_t c = i < V ? i : V - 1;
            const float v = (DT == kF32) ? ((const float*)rowp)[c] : bf16_to_float(((const uint16_t*)rowp)[c]);
            x[e] = i < V ? v : -INFINITY;
        }
    }
}

// Calls f(i0, x[4]) for every 4-token group of a row read from global memory.
template <int DT, class F>
__device__ __forceinline__ void row_groups(const Params& p, const void* rowp, F&& f)
{
    const int64_t ng = (p.V + 3) >> 2;
    for (int64_t g = threadIdx.x; g < ng; g += kThreads) {
        float x[4];
        load4<DT>(rowp, g << 2, p.V, p.vec_in, x);
        f(g << 2, x);
    }
}

// ---------------------------------------------------------------------------
// Cross-workgroup traffic.  Everything one workgroup publishes for another is
// written with device-coherent stores and read with device-coherent loads
// (relaxed agent-scope atomics: `sc1` accesses that bypass the per-XCD
// caches), so no cache-wide writeback or invalidate is ever needed.  Before a
// workgroup signals, every wave waits until its own stores have completed
// (s_waitcnt 0), and the signal is an atomic performed after that.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void put(T* p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T>
__device__ __forceinline__ T get(const T* p)
{
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bulk coherent traffic goes through buffer instructions carrying the same
// device-coherence bit (sc1) as the atomics above, but without the
// per-access waits the compiler attaches to atomics, so many loads can be in
// flight at once.  A resource covers up to 2 GB from `base`.
constexpr int kSC1 = 16;  // cache-policy bits: device-coherent (sc1)
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t join64(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent(const void* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ uint32_t cload32(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSC1);
}
__device__ __forceinline__ uint64_t cload64(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSC1);
    return ((uint64_t)v.y << 32) | v.x;
}
__device__ __forceinline__ u32x4v cload128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1);
}
__device__ __forceinline__ void cstore32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kSC1);
}
__device__ __forceinline__ void cstore128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4v v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSC1);
}
__device__ __forceinline__ void cstore64(__amdgpu_buffer_rsrc_t r, uint32_t off, uint64_t v)
{
    u32x2v w;
    w.x = (uint32_t)v;
    w.y = (uint32_t)(v >> 32);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kSC1);
}

// Every wave of the workgroup waits for its outstanding memory operations,
// then the workgroup synchronises: afterwards all its stores are complete.
__device__ __forceinline__ void drain_and_sync()
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Per-row barrier in the workspace (sense-reversing: the last arrival leaves
// the count at zero, and the last arriver bumps the generation the others
// wait on once its merge is published).
// ---------------------------------------------------------------------------
struct BarrierShared {
    uint32_t last, g0, timeout;
};

__device__ __forceinline__ bool barrier_arrive(RowCtl* c, uint32_t K, uint64_t epoch, BarrierShared& bs)
{
    drain_and_sync();
    if (threadIdx.x == 0) {
        const uint32_t g0 = get(&c->gen);
        // The arrival word is (epoch << 8) | count.  The first arrival of a
        // call finds another epoch there and installs (epoch, 1) by CAS; every
        // other arrival is one atomic add.
        uint32_t n = 0;
        uint64_t v = get(&c->arrive);
        if ((v >> 8) != epoch &&
            __hip_atomic_compare_exchange_strong(&c->arrive, &v, (epoch << 8) | 1u, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            n = 1;
        if (n == 0) {
            const uint64_t old =
                __hip_atomic_fetch_add(&c->arrive, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            n = (uint32_t)(old & 0xFFu) + 1u;
        }
        if (n == K) put(&c->arrive, epoch << 8);  // nobody arrives again before the release
        bs.g0 = g0;
        bs.last = (n == K) ? 1u : 0u;
        bs.timeout = 0;
    }
    __syncthreads();
    return bs.last != 0;
}

// Called by every thread of the last arriver once its merge is published.
__device__ __forceinline__ void barrier_release(RowCtl* c)
{
    drain_and_sync();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(&c->gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of a workgroup that arrived but was not last.  Returns false
// if the wait timed out; with give_up it gives up at once, without looking
// (the failure path, driven from the host by tests).
__device__ __forceinline__ bool barrier_wait(RowCtl* c, BarrierShared& bs, bool give_up)
{
    if (threadIdx.x == 0) {
        uint32_t n = 0;
        if (give_up) bs.timeout = 1;
        while (!give_up && get(&c->gen) == bs.g0) {
            __builtin_amdgcn_s_sleep(1);
            if (++n > kSpinLimit) {
                bs.timeout = 1;
                break;
            }
        }
    }
    __syncthreads();
    return bs.timeout == 0;
}

// ---------------------------------------------------------------------------
// Row state shared by the phases.
// ---------------------------------------------------------------------------
struct RowState {
    uint32_t mode;
    float m;
    uint32_t cbin;
    uint64_t tc;
    double a_above, s_total, s_keep;
    uint32_t token, count, cut_key;
};

// Mode of a row once its max is known (before any histogram).
__device__ __forceinline__ uint32_t first_mode(bool bad, float m, float T, float P, float MP, int K, bool want_probs)
{
    if (bad || T != T || P != P || MP != MP || !(m > -INFINITY)) return kModeError;
    if (T <= 0.0f) return kModeGreedy;
    if (K > 0 || (P > 0.0f && P < 1.0f) || (P >= 1.0f && want_probs)) return kModeHist;
    return P >= 1.0f ? kModeAll : kModeTop;
}

struct RowParams {
    float T, P, MP;
    int K;
};

// Row b's race key: its own seed when the call gives one per row (a
// per-request seed, "Top-p (Nucleus) Sampling, in depth", "Logprobs,
// speculative decoding and reproducibility").
__device__ __forceinline__ void use_row_key(Params& p, int64_t b)
{
    if (p.seeds) {
        const uint64_t s = p.seeds[b];
        p.seed_lo = (uint32_t)s;
        p.seed_hi = (uint32_t)(s >> 32);
    }
}

// Whether the call wants the renormalised distribution in any form.
__device__ __forceinline__ bool wants_dist(const Params& p) { return p.out_probs || p.out_logprobs; }

__device__ __forceinline__ RowParams row_params(const Params& p, int64_t b)
{
    RowParams r;
    r.T = p.temperature[b];
    r.P = p.top_p[b];
    r.MP = p.min_p ? p.min_p[b] : 0.0f;
    r.K = p.top_k ? p.top_k[b] : 0;
    return r;
}

// Rows whose histogram the parameters alone call for, before the max is
// known: a histogram is needed (first_mode would say kModeHist for any finite
// max) and min-p is off, so every finite token survives whatever the max.
__device__ __forceinline__ bool hist_before_max(const RowParams& rp, bool want_probs)
{
    if (!(rp.T > 0.0f) || rp.P != rp.P || rp.MP != rp.MP) return false;
    if (rp.MP > 0.0f && rp.T != INFINITY) return false;
    return rp.K > 0 || (rp.P > 0.0f && rp.P < 1.0f) || (rp.P >= 1.0f && want_probs);
}

struct RaceAcc {
    uint64_t best;
    uint32_t count, minkey;
    __device__ void init() { best = 0; count = 0; minkey = 0xFFFFFFFFu; }
};

// The exact race score e_i / E_i of one token (e from the compensated
// tempered weight, E from the token's Philox word).  Every path computes a
// winner's score with this one function, so all paths agree bit for bit; the
// hot loops only reach it for the few tokens that pass race_group's screen.
__device__ __attribute__((noinline)) float exact_score(float x, float m, float T, float invT, uint32_t word)
{
    return tempered_weight(x, m, T, invT) / exp1_from_word(word);
}

__device__ __forceinline__ uint32_t philox_word(const uint4& w4, uint32_t j)
{
    return j == 0 ? w4.x : j == 1 ? w4.y : j == 2 ? w4.z : w4.w;
}

// Race G groups of four consecutive tokens (group g starts at token i0[g];
// keep[g][j] marks the kept ones).  `scored` is false for greedy rows, where
// every kept token scores 1 so that the lowest index wins.  sstar is this
// lane's best exact score so far.  `track_min` off skips the smallest kept
// key: a row with crossing-bin candidates always keeps the top level of that
// bin, below every surely kept token, so its resolver finds that key.  Several groups per call let the Philox
// rounds of different groups interleave.
//
// The screen.  A token can reach sstar only if e/E >= sstar, i.e.
// E <= e/sstar; and E = -ln u >= w = 1 - u.  So a token with
// log2 w > log2 e - log2 sstar cannot reach sstar; the test runs in log2
// units, with no transcendental per token.  Both sides are bounded so that
// the test can only err towards scoring a token exactly:
//  - L, a lower bound of log2 w: w >= n 2^-32 with n = ~word, and for the
//    float nf of n, log2 nf >= bits(nf) 2^-23 - 127 (log2(1 + f) >= f on
//    [0, 1)), so L = bits(nf) 2^-23 - 159 - 5e-5 <= log2 w, the 5e-5
//    covering the roundings of n, of bits(nf) to a float and of the fused
//    add (together below 1.3e-5);
//  - R, an upper bound of log2 e - log2 sstar = (x - m) c - log2 sstar,
//    c = log2(e) / T, formed as fma(x - m, c, -log2 sstar + 2e-3): its
//    roundings and the hardware log2 stay below 1e-4, so R exceeds the
//    exact value by at least 1.9e-3 (a factor 1.0013 in the score).
// A token is rejected only when L > R, i.e. when its exact score is below
// sstar / 1.0013; the exact scorer's own error (about 1e-7 relative) cannot
// lift such a token to sstar, so no token that can reach sstar is dropped,
// ties included.  The bound w <= E is loose only when w is large, i.e. only
// for tokens whose e is a sizeable share of sstar; the many small tokens of
// a wide nucleus pass only when u is within e/sstar of 1, where w and E
// agree.
template <int G>
__device__ __forceinline__ void race_groups(const Params& p, int64_t b, bool scored, const RowModel& r, float c_log2e,
                                            const uint32_t i0[G], const float x[G][4], const bool keep[G][4],
                                            RaceAcc& acc, float& sstar, bool track_min = true)
{
    uint32_t km[G];
    bool any = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        km[g] = (keep[g][0] ? 1u : 0u) | (keep[g][1] ? 2u : 0u) | (keep[g][2] ? 4u : 0u) | (keep[g][3] ? 8u : 0u);
        any |= km[g] != 0;
    }
    if (!any) return;
#pragma unroll
    for (int g = 0; g < G; ++g) acc.count += (uint32_t)__builtin_popcount(km[g]);
    if (track_min) {  // uniform
        float xm = INFINITY;  // kept tokens are finite: a compare and a select do
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) xm = (keep[g][j] & (x[g][j] < xm)) ? x[g][j] : xm;
        const uint32_t kmin = order_key(xm);
        acc.minkey = kmin < acc.minkey ? kmin : acc.minkey;
    }
    if (!scored) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (!km[g]) continue;
            const uint64_t pk = race_pack(1.0f, i0[g] + (uint32_t)__builtin_ctz(km[g]));
            acc.best = pk > acc.best ? pk : acc.best;
        }
        return;
    }
    uint4 w4[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        w4[g] = philox4x32_10(make_uint4(i0[g] >> 2, (uint32_t)b, p.step_lo, p.step_hi), p.seed_lo, p.seed_hi);
    // q = -log2 sstar + margin (R errs high); with no score yet (sstar = 0)
    // every kept token passes.
    const float q = sstar > 0.0f ? -__builtin_amdgcn_logf(sstar) + 2e-3f : INFINITY;
    // Computed for every token and masked afterwards: no branches.  Tokens
    // go in from the last, so token 4 g + j's verdict ends at bit 4 g + j.
    uint32_t rej = 0, kall = 0;
#pragma unroll
    for (int g = G - 1; g >= 0; --g) {
        kall = (kall << 4) | km[g];
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            const float R = fmaf(x[g][j] - r.m, c_log2e, q);
            const float nf = (float)(~philox_word(w4[g], (uint32_t)j));
            const float L = fmaf((float)__float_as_uint(nf), 0x1p-23f, -159.00005f);
            rej = shift_in_gt(rej, L, R);
        }
    }
    uint32_t pass = kall & ~rej;
    while (pass) {
        const uint32_t k = (uint32_t)__builtin_ctz(pass);
        pass &= pass - 1u;
        const uint32_t g = k >> 2, j = k & 3u;
        uint32_t gi0 = i0[0];
        float gx = x[0][0];
        uint32_t word = w4[0].x;
#pragma unroll
        for (int q = 0; q < G; ++q)
            if ((uint32_t)q == g) {
                gi0 = i0[q];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if ((uint32_t)jj == j) {
                        gx = x[q][jj];
                        word = philox_word(w4[q], (uint32_t)jj);
                    }
            }
        const float s = exact_score(gx, r.m, r.T, r.invT, word);
        const uint64_t pk = race_pack(s, gi0 + j);
        acc.best = pk > acc.best ? pk : acc.best;
        sstar = fmaxf(sstar, s);
    }
}

// One group (the split-row kernel's register-resident chunk).
__device__ __forceinline__ void race_group(const Params& p, int64_t b, bool scored, const RowModel& r, float c_log2e,
                                           uint32_t i0, const float x[4], const bool keep[4], RaceAcc& acc,
                                           float& sstar, bool track_min)
{
    const uint32_t i0s[1] = {i0};
    float xs[1][4];
    bool ks[1][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        xs[0][j] = x[j];
        ks[0][j] = keep[j];
    }
    race_groups<1>(p, b, scored, r, c_log2e, i0s, xs, ks, acc, sstar, track_min);
}

// Race one token by index (resolver candidates).
__device__ __forceinline__ void race_one(const Params& p, int64_t b, const RowModel& r, uint32_t key, uint32_t idx,
                                         RaceAcc& acc)
{
    const uint4 w4 = philox4x32_10(make_uint4(idx >> 2, (uint32_t)b, p.step_lo, p.step_hi), p.seed_lo, p.seed_hi);
    const float s = exact_score(key_value(key), r.m, r.T, r.invT, philox_word(w4, idx & 3));
    const uint64_t pk = race_pack(s, idx);
    acc.best = pk > acc.best ? pk : acc.best;
    acc.count += 1;
    acc.minkey = key < acc.minkey ? key : acc.minkey;
}

// race_one behind race_groups' screen against a bound score s0, passed as
// k0 = (1 + 1e-4) / ((1 - 1e-4) s0) (INFINITY for no bound): a token whose
// 1 - u exceeds e_hat k0 scores below s0 and cannot win; it is counted and
// its key kept, but not scored.
__device__ __forceinline__ void race_one_screened(const Params& p, int64_t b, const RowModel& r, uint32_t key,
                                                  uint32_t idx, RaceAcc& acc, float c_log2e, float k0)
{
    const uint4 w4 = philox4x32_10(make_uint4(idx >> 2, (uint32_t)b, p.step_lo, p.step_hi), p.seed_lo, p.seed_hi);
    const uint32_t word = philox_word(w4, idx & 3);
    const float x = key_value(key);
    const float e_hat = __builtin_amdgcn_exp2f((x - r.m) * c_log2e);
    const float w = fmaf((float)(0xFFFFFFFFu - word), 0x1p-32f, 0x1p-33f);
    if (!(w > e_hat * k0)) {
        const float s = exact_score(x, r.m, r.T, r.invT, word);
        const uint64_t pk = race_pack(s, idx);
        acc.best = pk > acc.best ? pk : acc.best;
    }
    acc.count += 1;
    acc.minkey = key < acc.minkey ? key : acc.minkey;
}

// The smallest finite logit whose bin is < c (c >= 1).  Bins fall as logits
// rise (the row max is in bin 0), so over order keys this is the boundary
// between keys with bin >= c and keys with bin < c.  The search starts from
// the estimate (A - c + 1)/s (the lower edge of bin c - 1), gallops in key steps until it brackets the boundary
// and bisects the bracket: the same answer as a bisection over all keys, in a
// few evaluations.
__device__ __forceinline__ float lowest_in_bins_below(const RowModel& r, uint32_t c)
{
    const uint32_t kmin = order_key(-3.4028234663852886e38f), kmax = order_key(r.m);
    auto below = [&](uint32_t key) { return bin_of(r, key_value(key)) < c; };
    if (below(kmin)) return key_value(kmin);  // also every row with s = 0 (T = +inf)
    const float est = (float)((r.A - (double)c + 1.0) / r.L.s);
    uint32_t k = order_key(est > -3.4028234663852886e38f ? est : -3.4028234663852886e38f);
    k = k < kmin ? kmin : (k > kmax ? kmax : k);
    uint32_t lo, hi;  // below(lo) is false, below(hi) is true
    // Steps double up to 2^31 and then stay there, so every step moves and
    // the gallop reaches kmin (not below) or kmax (below: the max is in bin
    // 0) from any start.
    if (below(k)) {
        hi = k;
        for (uint32_t step = 1;; step = step < 0x80000000u ? step << 1 : step) {
            lo = (hi - kmin > step) ? hi - step : kmin;
            if (!below(lo)) break;
            hi = lo;
        }
    } else {
        lo = k;
        for (uint32_t step = 1;; step = step < 0x80000000u ? step << 1 : step) {
            hi = (kmax - lo > step) ? lo + step : kmax;
            if (below(hi)) break;
            lo = hi;
        }
    }
    while (hi - lo > 1) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (below(mid)) hi = mid; else lo = mid;
    }
    return key_value(hi);
}

// Thresholds on the logit that classify the tokens of a row after its mode is
// known: surely kept iff x >= keep_lo; candidate iff cand_lo <= x < keep_lo.
struct Classes {
    float keep_lo, cand_lo;
};

__device__ __forceinline__ Classes classify(const RowModel& r, const RowState& st)
{
    Classes c;
    c.keep_lo = INFINITY;
    c.cand_lo = INFINITY;
    const float floor_ = fmaxf(r.tmp, -3.4028234663852886e38f);  // survivors: finite and >= tmp
    switch (st.mode) {
    case kModeGreedy:
    case kModeTop: c.keep_lo = st.m; break;
    case kModeAll: c.keep_lo = floor_; break;
    case kModeP:
        if (st.cbin > 0) c.keep_lo = fmaxf(floor_, lowest_in_bins_below(r, st.cbin));
        c.cand_lo = (st.cbin + 1 < (uint32_t)kBins) ? fmaxf(floor_, lowest_in_bins_below(r, st.cbin + 1)) : floor_;
        break;
    case kModeK:
        c.cand_lo = (st.cbin + 1 < (uint32_t)kBins) ? fmaxf(floor_, lowest_in_bins_below(r, st.cbin + 1)) : floor_;
        break;
    default: break;
    }
    return c;
}

struct ResolveShared {
    SelectShared sel;
    uint64_t red64[kMaxWaves];
    uint32_t red32[kMaxWaves];
    uint32_t red32b[kMaxWaves];
};

// Merge partial race accumulators of the workgroup (all threads return the
// merge): wave reductions, then one exchange through LDS.
template <int NT>
__device__ __forceinline__ RaceAcc block_race(RaceAcc a, ResolveShared& rs)
{
    constexpr int W = NT / kWave;
    a.best = wave_reduce(a.best, MaxU64());
    a.count = wave_reduce(a.count, SumU32());
    a.minkey = wave_reduce(a.minkey, MinU32());
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) {
        rs.red64[w] = a.best;
        rs.red32[w] = a.count;
        rs.red32b[w] = a.minkey;
    }
    __syncthreads();
    RaceAcc o;
    o.best = rs.red64[0];
    o.count = rs.red32[0];
    o.minkey = rs.red32b[0];
#pragma unroll
    for (int i = 1; i < W; ++i) {
        o.best = rs.red64[i] > o.best ? rs.red64[i] : o.best;
        o.count += rs.red32[i];
        o.minkey = rs.red32b[i] < o.minkey ? rs.red32b[i] : o.minkey;
    }
    return o;
}

// The last step of a row: given the merged race partial of the surely kept
// tokens (`part`), the row's classes and a way to visit the candidates
// (`visit(fn(key, idx))`, every token with cl.cand_lo <= x < cl.keep_lo),
// find the exact cut, race the kept candidates and fill st.token / count /
// cut_key / s_keep.  All NT threads; uniform control flow.
template <int NT, class Visit>
__device__ __forceinline__ void resolve_row(const Params& p, int64_t b, const RowModel& r, const RowParams& rp, RowState& st,
                            RaceAcc part, const Classes& cl, Visit visit, ResolveShared& rs)
{
    // Keys every candidate lies between (they bound the radix search).
    const uint32_t key_lo = order_key(cl.cand_lo);
    const uint32_t key_hi = cl.keep_lo < INFINITY ? order_key(cl.keep_lo) - 1u : order_key(st.m);
    if (st.mode == kModeError) {
        st.token = 0xFFFFFFFFu;
        st.count = 0;
        st.cut_key = 0;
        st.s_keep = 0.0;
        return;
    }
    if (st.mode == kModeGreedy) {
        st.token = ~(uint32_t)part.best;
        st.count = 1;
        st.cut_key = order_key(st.m);
        st.s_keep = 1.0;
        return;
    }
    RaceAcc acc = part;
    if (st.mode == kModeTop) {
        // Every top-level token weighs what the max does.
        st.s_keep = (double)acc.count * ((double)bin_fx(r, st.m) * (1.0 / kFx));
    } else if (st.mode == kModeAll) {
        st.s_keep = st.s_total;
    } else if (st.mode == kModeP) {
        const uint64_t tc = st.tc;
        const SelectResult sr = select_level<NT>(
            [&](auto&& fn) {
                visit([&](uint32_t key, uint32_t) { fn(key, (uint64_t)bin_fx(r, key_value(key))); });
            },
            [&](uint64_t) { return tc; }, rs.sel, key_lo, key_hi);
        const uint32_t cut = sr.level;
        RaceAcc c;
        c.init();
        // Kept candidates are screened against the surely kept tokens' best
        // score (race_groups' screen): one that cannot reach it is counted
        // without its exact score.
        const float s0 = __uint_as_float((uint32_t)(part.best >> 32));
        const float k0 = s0 > 0.0f ? __builtin_amdgcn_rcpf(s0) * (1.0001f / (1.0f - 1e-4f)) : INFINITY;
        const float c_log2e = r.invT * 1.4426950408889634f;
        visit([&](uint32_t key, uint32_t idx) {
            if (key >= cut) race_one_screened(p, b, r, key, idx, c, c_log2e, k0);
        });
        c = block_race<NT>(c, rs);
        acc.best = c.best > acc.best ? c.best : acc.best;
        acc.count += c.count;
        acc.minkey = c.minkey < acc.minkey ? c.minkey : acc.minkey;
        st.s_keep = st.a_above + edge_weight(r, (int)st.cbin) * ((double)(sr.above + sr.at) * (1.0 / kFx));
    } else {  // kModeK: top-k binds; every candidate decision is taken here
        const uint64_t kk = (uint64_t)rp.K;
        const SelectResult tk = select_level<NT>(
            [&](auto&& fn) { visit([&](uint32_t key, uint32_t) { fn(key, (uint64_t)1); }); },
            [&](uint64_t) { return kk; }, rs.sel, key_lo, key_hi);
        uint32_t cut = tk.level;
        if (rp.P <= 0.0f) {
            cut = order_key(st.m);
        } else if (rp.P < 1.0f) {
            const uint32_t vk = tk.level;
            const float P = rp.P;
            const SelectResult sp = select_level<NT>(
                [&](auto&& fn) {
                    visit([&](uint32_t key, uint32_t) {
                        if (key >= vk) fn(key, fixed40(r, bin_token(r, key_value(key))));
                    });
                },
                [&](uint64_t total) { return ceil_p_times(P, total); }, rs.sel, vk, key_hi);
            cut = sp.level;
        }
        RaceAcc c;
        c.init();
        uint64_t kept_w = 0;
        visit([&](uint32_t key, uint32_t idx) {
            if (key >= cut) {
                race_one(p, b, r, key, idx, c);
                kept_w += fixed40(r, bin_token(r, key_value(key)));
            }
        });
        c = block_race<NT>(c, rs);
        kept_w = block_reduce<NT>(kept_w, SumU64(), rs.red64);
        acc = c;
        st.s_keep = (double)kept_w * 0x1p-40;
    }
    st.token = ~(uint32_t)acc.best;
    st.count = acc.count;
    st.cut_key = acc.minkey;
}

__device__ __forceinline__ void write_outputs(const Params& p, int64_t b, const RowState& st)
{
    if (threadIdx.x != 0) return;
    if (st.mode == kModeError) {
        p.out_token[b] = -1;
        p.out_count[b] = 0;
        if (p.out_min_kept) p.out_min_kept[b] = __uint_as_float(0x7FC00000u);
        return;
    }
    p.out_token[b] = (int32_t)st.token;
    p.out_count[b] = (int32_t)st.count;
    if (p.out_min_kept) p.out_min_kept[b] = key_value(st.cut_key);
}

// Per-bin factors edge(j) * 2^-31 / S_keep for the probability pass.
template <int NT>
__device__ __forceinline__ void prob_factors(const RowModel& r, const RowState& st, float* factor)
{
    for (int j = threadIdx.x; j < kBins; j += NT)
        factor[j] = (st.s_keep > 0.0) ? (float)(edge_weight(r, j) * (1.0 / kFx) / st.s_keep) : 0.0f;
    __syncthreads();
}

// ln S_keep with S_keep = sum of exp((x_i - m)/T) over the kept tokens, split
// into two floats.  s_keep is held in the bin model's units (weights measured
// from the lattice point (A + 1)/s above the max, a common factor
// exp((m s - A - 1) w) below the true weights), so
// ln S_keep = ln s_keep + (A + 1 - m s) w.
struct LogNorm {
    float hi, lo;
};

__device__ __forceinline__ LogNorm log_norm(const RowModel& r, const RowState& st)
{
#pragma clang fp contract(off)
    LogNorm n;
    n.hi = n.lo = 0.0f;
    if (st.mode == kModeError || st.mode == kModeGreedy || !(st.s_keep > 0.0)) return n;
    const double l = log(st.s_keep) + ((r.A + 1.0) - (double)r.m * r.L.s) * r.L.w;
    n.hi = (float)l;
    n.lo = (float)(l - (double)n.hi);
    return n;
}

// Log-probability of token i (logit x) in the renormalised kept distribution
// (the processed distribution: -inf outside the nucleus, "Top-p (Nucleus)
// Sampling, in depth", "Logprobs, speculative decoding and reproducibility"):
// (x - m)/T - ln S_keep, with (x - m)/T carried to about one extra word as in
// tempered_weight; 0 / -inf on greedy rows, NaN on error rows.
__device__ __forceinline__ float logprob_of(uint32_t mode, const RowModel& r, const RowState& st, const LogNorm& n,
                                            float x, int64_t i)
{
#pragma clang fp contract(off)
    if (mode == kModeError) return __builtin_nanf("");
    if (mode == kModeGreedy) return (uint32_t)i == st.token ? 0.0f : -INFINITY;
    if (!(survives(r, x) && order_key(x) >= st.cut_key)) return -INFINITY;
    if (r.invT == 0.0f) return -n.hi - n.lo;  // T = +inf: every kept token weighs the same
    const float s = x - r.m;
    const float q = s * r.invT;
    const float bb = s - x;
    const float err = (x - (s - bb)) + (-r.m - bb);  // x - m == s + err exactly
    const float rem = fmaf(-q, r.T, s);              // s - q*T exactly
    const float lo = (rem + err) * r.invT;
    return (q - n.hi) + (lo - n.lo);
}

__device__ __forceinline__ float prob_of(uint32_t mode, const RowModel& r, const RowState& st, const float* factor,
                                         float x, int64_t i)
{
    if (mode == kModeError) return 0.0f;
    if (mode == kModeGreedy) return (uint32_t)i == st.token ? 1.0f : 0.0f;
    if (!(survives(r, x) && order_key(x) >= st.cut_key)) return 0.0f;
    const Binned t = bin_token(r, x);
    return (float)t.fx * factor[t.j];
}

// ---------------------------------------------------------------------------
// The split-row kernel.
// ---------------------------------------------------------------------------
struct TileShared {
    union {
        struct {
            uint64_t hm[kBins];
            uint32_t hc[kBins];
        } h;
        float factor[kBins];
        u32x2v cand[kCandLds];  // the row's candidates, staged for the resolver
    } u;
    ResolveShared rs;
    float redf[kThreads / kWave];
    int redi[kThreads / kWave];
    uint32_t red32[kThreads / kWave];
    BarrierShared bar;
    RowState st;
    uint32_t cand_base;
};

__device__ __forceinline__ RowState uniform(const RowState& a)
{
    RowState s;
    s.mode = uniform(a.mode);
    s.m = uniform(a.m);
    s.cbin = uniform(a.cbin);
    s.tc = uniform(a.tc);
    s.a_above = uniform(a.a_above);
    s.s_total = uniform(a.s_total);
    s.s_keep = uniform(a.s_keep);
    s.token = uniform(a.token);
    s.count = uniform(a.count);
    s.cut_key = uniform(a.cut_key);
    return s;
}

// Byte offsets of the published fields of RowCtl.
constexpr uint32_t kOffMode = 16, kOffM = 20, kOffCbin = 28, kOffCut = 32, kOffCount = 36,
                   kOffTc = 40, kOffAbove = 48, kOffStotal = 56, kOffSkeep = 64, kOffToken = 72, kOffCandN = 12;

static_assert(offsetof(RowCtl, cand_n) == kOffCandN && offsetof(RowCtl, mode) == kOffMode &&
                  offsetof(RowCtl, m) == kOffM &&
                  offsetof(RowCtl, cbin) == kOffCbin && offsetof(RowCtl, cut_key) == kOffCut &&
                  offsetof(RowCtl, count) == kOffCount && offsetof(RowCtl, tc) == kOffTc &&
                  offsetof(RowCtl, a_above) == kOffAbove && offsetof(RowCtl, s_total) == kOffStotal &&
                  offsetof(RowCtl, s_keep) == kOffSkeep && offsetof(RowCtl, token) == kOffToken,
              "RowCtl field offsets");

__device__ __forceinline__ void read_state(RowCtl* c, RowState& st)
{
    if (threadIdx.x == 0) {
        const __amdgpu_buffer_rsrc_t r = coherent(c);
        const u32x4v q1 = cload128(r, 16), q2 = cload128(r, 32), q3 = cload128(r, 48), q4 = cload128(r, 64);
        st.mode = q1.x;
        st.m = __uint_as_float(q1.y);
        st.cbin = q1.w;
        st.cut_key = q2.x;
        st.count = q2.y;
        st.tc = join64(q2.z, q2.w);
        st.a_above = __longlong_as_double((long long)join64(q3.x, q3.y));
        st.s_total = __longlong_as_double((long long)join64(q3.z, q3.w));
        st.s_keep = __longlong_as_double((long long)join64(q4.x, q4.y));
        st.token = q4.z;
    }
    __syncthreads();
}

__device__ __forceinline__ void timed_out(const Params& p, int64_t b)
{
    if (threadIdx.x == 0) p.out_token[b] = -2;
}

template <int DT>
__global__ __launch_bounds__(kThreads, 4) void tile_kernel(Params p, Work wk)
{
    __shared__ TileShared sh;
    const uint32_t K = (uint32_t)wk.K;
    const uint32_t grp = blockIdx.x / (8u * K), rem = blockIdx.x % (8u * K);
    const uint32_t chunk = rem >> 3;
    const int64_t b = (int64_t)grp * 8 + (rem & 7);
    if (b >= p.B) return;
    const int t = threadIdx.x;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    const int64_t base = (int64_t)chunk * kChunk;
    RowCtl* ctl = wk.ctl + b;
    const int64_t wg = b * K + chunk;
    const bool give_up = b == wk.give_up_row;
    use_row_key(p, b);
    const bool want_probs = wants_dist(p);  // probabilities or log-probabilities

    // ---- load the chunk into registers (token of x[4v+j]: lane0 + 1024 v + j)
    float x[kEPT];
    const uint32_t lane0 = (uint32_t)base + (uint32_t)t * 4u;
    load_chunk<DT, kEPT>(rowp, lane0, (uint32_t)base + kChunk, (uint32_t)p.V, p.vec_in, x);

    // ---- A: row max, NaN / +inf
    float lmax = -INFINITY;
    int bad = 0;
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
        const float v = x[e];
        bad |= !(v < INFINITY);  // NaN or +inf
        lmax = fmaxf(lmax, v);
    }
    lmax = block_reduce<kThreads>(lmax, MaxF(), sh.redf);
    bad = block_reduce<kThreads>(bad, OrI32(), sh.redi);
    if (t == 0) {
        u32x4v a;
        a.x = __float_as_uint(lmax);
        a.y = (uint32_t)bad;
        a.z = 0;
        a.w = 0;
        cstore128(coherent(wk.slot_a + wg), 0, a);
    }
    const RowParams rp = row_params(p, b);

    if (barrier_arrive(ctl, K, wk.epoch, sh.bar)) {
        float m = -INFINITY;
        int e = 0;
        const __amdgpu_buffer_rsrc_t ra = coherent(wk.slot_a + b * K);
        for (uint32_t k = t; k < K; k += kThreads) {
            const u32x4v a = cload128(ra, k * 16);
            m = fmaxf(m, __uint_as_float(a.x));
            e |= (int)a.y;
        }
        m = block_reduce<kThreads>(m, MaxF(), sh.redf);
        e = block_reduce<kThreads>(e, OrI32(), sh.redi);
        if (t == 0) {
            const __amdgpu_buffer_rsrc_t rc = coherent(ctl);
            cstore32(rc, kOffM, __float_as_uint(m));
            cstore32(rc, kOffMode, first_mode(e != 0, m, rp.T, rp.P, rp.MP, rp.K, want_probs));
        }
        barrier_release(ctl);
    } else if (!barrier_wait(ctl, sh.bar, give_up)) {
        timed_out(p, b);
        return;
    }
    read_state(ctl, sh.st);
    RowState st = uniform(sh.st);
    RowModel model = {};
    if (st.mode >= kModeTop) model = uniform(make_model(st.m, rp.T, rp.MP));

    // ---- B: bin histogram of the survivors
    if (st.mode == kModeHist) {
        const bool counts = rp.K > 0;
        for (int i = t; i < kBins; i += kThreads) {
            sh.u.h.hm[i] = 0;
            sh.u.h.hc[i] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
            if (survives(model, x[e])) {
                const Binned bt = bin_token(model, x[e]);
                const uint32_t j = bt.j;
                atomicAdd((unsigned long long*)&sh.u.h.hm[j], (unsigned long long)bt.fx);
                if (counts) atomicAdd(&sh.u.h.hc[j], 1u);
            }
        }
        __syncthreads();
        const __amdgpu_buffer_rsrc_t rh = coherent(wk.slot_h + b * K * kBins);
        const __amdgpu_buffer_rsrc_t rcn = coherent(wk.slot_c + b * K * kBins);
        for (int i = t; i < kBins; i += kThreads) {
            cstore64(rh, (uint32_t)((chunk * kBins + i) * 8), sh.u.h.hm[i]);
            if (counts) cstore32(rcn, (uint32_t)((chunk * kBins + i) * 4), sh.u.h.hc[i]);
        }
        if (barrier_arrive(ctl, K, wk.epoch, sh.bar)) {
            // Every thread takes 16-byte pieces (two bins) of every slot, eight
            // loads in flight at a time, and adds them into LDS: the K slots are
            // read in parallel rather than one round trip after another.
            for (int i = t; i < kBins; i += kThreads) {
                sh.u.h.hm[i] = 0;
                sh.u.h.hc[i] = 0;
            }
            __syncthreads();
            const uint32_t pieces = K * (kBins / 2);
            for (uint32_t q0 = t; q0 < pieces; q0 += kMergeBatch * kThreads) {
                u32x4v v[kMergeBatch];
#pragma unroll
                for (int u = 0; u < kMergeBatch; ++u) {
                    const uint32_t q = q0 + u * kThreads;
                    v[u] = cload128(rh, (q < pieces ? q : 0) * 16);
                }
#pragma unroll
                for (int u = 0; u < kMergeBatch; ++u) {
                    const uint32_t q = q0 + u * kThreads;
                    if (q < pieces) {
                        const uint32_t i = (q % (kBins / 2)) * 2;
                        if (v[u].x | v[u].y) atomicAdd((unsigned long long*)&sh.u.h.hm[i], (unsigned long long)join64(v[u].x, v[u].y));
                        if (v[u].z | v[u].w) atomicAdd((unsigned long long*)&sh.u.h.hm[i + 1], (unsigned long long)join64(v[u].z, v[u].w));
                    }
                }
            }
            if (counts) {
                const uint32_t cpieces = K * (kBins / 4);
                for (uint32_t q0 = t; q0 < cpieces; q0 += kMergeBatch * kThreads) {
                    u32x4v v[kMergeBatch];
#pragma unroll
                    for (int u = 0; u < kMergeBatch; ++u) {
                        const uint32_t q = q0 + u * kThreads;
                        v[u] = cload128(rcn, (q < cpieces ? q : 0) * 16);
                    }
#pragma unroll
                    for (int u = 0; u < kMergeBatch; ++u) {
                        const uint32_t q = q0 + u * kThreads;
                        if (q < cpieces) {
                            const uint32_t i = (q % (kBins / 4)) * 4;
                            if (v[u].x) atomicAdd(&sh.u.h.hc[i], v[u].x);
                            if (v[u].y) atomicAdd(&sh.u.h.hc[i + 1], v[u].y);
                            if (v[u].z) atomicAdd(&sh.u.h.hc[i + 2], v[u].z);
                            if (v[u].w) atomicAdd(&sh.u.h.hc[i + 3], v[u].w);
                        }
                    }
                }
            }
            __syncthreads();
            const Decision d = decide(model, sh.u.h.hm, counts ? sh.u.h.hc : nullptr, rp.K, rp.P);
            if (t == 0) {
                const __amdgpu_buffer_rsrc_t rc = coherent(ctl);
                put(&ctl->cand_n, 0u);  // the candidates of this call are appended after this barrier
                cstore32(rc, kOffMode, d.mode);
                cstore32(rc, kOffCbin, d.cbin);
                cstore64(rc, kOffTc, d.tc);
                cstore64(rc, kOffAbove, (uint64_t)__double_as_longlong(d.a_above));
                cstore64(rc, kOffStotal, (uint64_t)__double_as_longlong(d.s_total));
            }
            barrier_release(ctl);
        } else if (!barrier_wait(ctl, sh.bar, give_up)) {
            timed_out(p, b);
            return;
        }
        read_state(ctl, sh.st);
        st = uniform(sh.st);
    }

    // ---- C: race the surely kept tokens, compact the candidates
    const Classes cl = classify(model, st);
    const float keep_lo = uniform(cl.keep_lo), cand_lo = uniform(cl.cand_lo);
    const bool scored = st.mode != kModeGreedy;
    const float c_log2e = uniform(model.invT * 1.4426950408889634f);
    RaceAcc acc;
    acc.init();
    float sstar = 0.0f;
    uint32_t ncand = 0;
    const bool has_cands = st.mode == kModeP || st.mode == kModeK;
#pragma unroll
    for (int v = 0; v < kEPT / 4; ++v) {
        const uint32_t i0 = lane0 + (uint32_t)v * (kThreads * 4);
        bool keep[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            keep[j] = x[4 * v + j] >= keep_lo;
            ncand += (x[4 * v + j] >= cand_lo && !keep[j]) ? 1u : 0u;
        }
        race_group(p, b, scored, model, c_log2e, i0, &x[4 * v], keep, acc, sstar, !has_cands);
        if (scored) sstar = wave_reduce(sstar, MaxF());
    }
    if (has_cands) {
        const uint64_t excl = block_exclusive_sum<kThreads>((uint64_t)ncand, sh.rs.red64);
        const uint32_t total = (uint32_t)block_reduce<kThreads>((uint64_t)ncand, SumU64(), sh.rs.red64);
        if (t == 0) sh.cand_base = total ? atomicAdd(&ctl->cand_n, total) : 0u;
        __syncthreads();
        uint32_t pos = sh.cand_base + (uint32_t)excl;
        const __amdgpu_buffer_rsrc_t rk = coherent(wk.cand + b * kCap);
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
            if (x[e] >= cand_lo && x[e] < keep_lo) {
                if (pos < (uint32_t)kCap)
                    cstore64(rk, pos * 8,
                             ((uint64_t)(lane0 + (uint32_t)(e >> 2) * (kThreads * 4) + (uint32_t)(e & 3)) << 32) |
                                 order_key(x[e]));
                ++pos;
            }
        }
    }
    acc = block_race<kThreads>(acc, sh.rs);
    if (t == 0) {
        u32x4v q;
        q.x = (uint32_t)acc.best;
        q.y = (uint32_t)(acc.best >> 32);
        q.z = acc.count;
        q.w = acc.minkey;
        cstore128(coherent(wk.slot_r + wg), 0, q);
    }

    if (barrier_arrive(ctl, K, wk.epoch, sh.bar)) {
        RaceAcc part;
        part.init();
        const __amdgpu_buffer_rsrc_t rr = coherent(wk.slot_r + b * K);
        for (uint32_t k = t; k < K; k += kThreads) {
            const u32x4v q = cload128(rr, k * 16);
            const uint64_t qb = join64(q.x, q.y);
            part.best = qb > part.best ? qb : part.best;
            part.count += q.z;
            part.minkey = q.w < part.minkey ? q.w : part.minkey;
        }
        part = block_race<kThreads>(part, sh.rs);
        uint32_t n = 0;
        if (has_cands) {
            if (t == 0) sh.cand_base = get(&ctl->cand_n);
            __syncthreads();
            n = sh.cand_base;
        }
        if (n <= (uint32_t)kCandLds) {
            // One pass over the list with four loads in flight per thread puts
            // it in LDS; the resolver's passes then read LDS.
            const __amdgpu_buffer_rsrc_t rk = coherent(wk.cand + b * kCap);
            for (uint32_t i0 = t; i0 < n; i0 += 4 * kThreads) {
                u32x2v c[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t i = i0 + u * kThreads;
                    c[u] = __builtin_amdgcn_raw_buffer_load_b64(rk, (i < n ? i : 0) * 8, 0, kSC1);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i0 + u * kThreads < n) sh.u.cand[i0 + u * kThreads] = c[u];
            }
            __syncthreads();
            resolve_row<kThreads>(p, b, model, rp, st,
                        part, cl, [&](auto&& fn) {
                            for (uint32_t i = t; i < n; i += kThreads) {
                                const u32x2v c = sh.u.cand[i];
                                fn(c.x, c.y);
                            }
                        },
                        sh.rs);
        } else if (n <= (uint32_t)kCap) {
            const __amdgpu_buffer_rsrc_t rk = coherent(wk.cand + b * kCap);
            resolve_row<kThreads>(p, b, model, rp, st,
                        part, cl, [&](auto&& fn) {
                            for (uint32_t i = t; i < n; i += kThreads) {
                                const u32x2v c = __builtin_amdgcn_raw_buffer_load_b64(rk, i * 8, 0, kSC1);
                                fn(c.x, c.y);
                            }
                        },
                        sh.rs);
        } else {  // the crossing bin overflowed the list: visit the row in global memory
            resolve_row<kThreads>(p, b, model, rp, st,
                        part, cl, [&](auto&& fn) {
                            row_groups<DT>(p, rowp, [&](int64_t i0, const float* xs) {
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    if (xs[j] >= cand_lo && xs[j] < keep_lo) fn(order_key(xs[j]), (uint32_t)(i0 + j));
                            });
                        },
                        sh.rs);
        }
        write_outputs(p, b, st);
        if (t == 0) {
            const __amdgpu_buffer_rsrc_t rc = coherent(ctl);
            cstore32(rc, kOffToken, st.token);
            cstore32(rc, kOffCount, st.count);
            cstore32(rc, kOffCut, st.cut_key);
            cstore64(rc, kOffSkeep, (uint64_t)__double_as_longlong(st.s_keep));
        }
        barrier_release(ctl);
        if (!want_probs) return;
        // The resolving workgroup re-reads its chunk so that its registers are
        // free for the resolver; the others write from registers below.
        if (p.out_probs && st.mode != kModeError && st.mode != kModeGreedy)
            prob_factors<kThreads>(model, st, sh.u.factor);
        const LogNorm ln = log_norm(model, st);
        for (int v = 0; v < kEPT / 4; ++v) {
            const int64_t i0 = base + ((int64_t)v * kThreads + t) * 4;
            float xs[4];
            load4<DT>(rowp, i0, p.V, p.vec_in, xs);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (i0 + j < p.V) {
                    if (p.out_probs) p.out_probs[b * p.V + i0 + j] = prob_of(st.mode, model, st, sh.u.factor, xs[j], i0 + j);
                    if (p.out_logprobs) p.out_logprobs[b * p.V + i0 + j] = logprob_of(st.mode, model, st, ln, xs[j], i0 + j);
                }
        }
        return;
    }
    if (!want_probs) return;
    if (!barrier_wait(ctl, sh.bar, give_up)) {
        timed_out(p, b);
        return;
    }
    read_state(ctl, sh.st);
    st = uniform(sh.st);

    // ---- probabilities / log-probabilities of this chunk, from registers
    if (p.out_probs && st.mode != kModeError && st.mode != kModeGreedy) prob_factors<kThreads>(model, st, sh.u.factor);
    const LogNorm ln = log_norm(model, st);
#pragma unroll
    for (int v = 0; v < kEPT / 4; ++v) {
        const uint32_t i0 = lane0 + (uint32_t)v * (kThreads * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i0 + j < (uint32_t)p.V) {
                if (p.out_probs)
                    p.out_probs[b * p.V + i0 + j] = prob_of(st.mode, model, st, sh.u.factor, x[4 * v + j], i0 + j);
                if (p.out_logprobs)
                    p.out_logprobs[b * p.V + i0 + j] = logprob_of(st.mode, model, st, ln, x[4 * v + j], i0 + j);
            }
    }
}

// ---------------------------------------------------------------------------
// One workgroup per row, every phase streamed from global memory.
// ---------------------------------------------------------------------------
}  // namespace nucleus
