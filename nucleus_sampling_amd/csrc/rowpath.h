// rowpath.h -- the sampler's kernels for batches large enough to give every
// row a CU of its own.
//
// row_kernel: one 1024-thread workgroup per row streams the row from global
//   memory once per pass, eight 16-byte loads in flight per thread:
//     1  row max, smallest finite logit, error flag  -> row mode, model
//     2  bin histogram of the survivors (LDS)          -> crossing bin (decide)
//   then either finishes the row itself (one more pass racing the surely kept
//   tokens and gathering the crossing bin's tokens into LDS, the resolver,
//   and an optional probability pass), or publishes the row's state for
//   race_kernel.
//
// race_kernel: the race pass split over chunks of 8192 tokens, one 256-thread
//   workgroup each, so a row that keeps most of its tokens (whose Philox
//   draws dominate) spreads over many CUs instead of holding one.  Each
//   chunk merges its race partial into the row's state with order-free
//   atomics (max of the packed score, sums, min) and appends its candidates
//   to the row's list; the chunk that finishes a row last resolves it.  No
//   workgroup ever waits for another.
//
// probs_kernel: the optional probability pass, chunked the same way.
//
// Every kernel uses the model's functions and nothing else to weigh tokens,
// so all paths take the same decisions, bit for bit.
#pragma once

#include "sampler.h"

namespace nucleus {

constexpr int kRowThreads = 1024;  // 16 waves: one workgroup per CU
constexpr int kRowUnroll = 8;      // 4-token groups per thread whose loads are in flight together
constexpr int kRowCand = 8192;     // crossing-bin candidates held in LDS
constexpr int kRaceQueue = 128;    // per-wave ring of 4-token groups waiting for the race
constexpr int kRaceThreads = 256;  // race_kernel / probs_kernel workgroups
constexpr int kRaceUnroll = 8;
constexpr int kRaceChunk = kRaceThreads * kRaceUnroll * 4;  // tokens per race_kernel workgroup

// One aligned 4-token group (f32: 16 bytes, bf16: 8 bytes) at group index g.
template <int DT, bool NTL>
__device__ __forceinline__ void load_group(const void* rowp, uint32_t g, float x[4])
{
    if (DT == kF32) {
        const f32x4* a = (const f32x4*)rowp + g;
        const f32x4 v = NTL ? __builtin_nontemporal_load(a) : *a;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else {
        const u32x2* a = (const u32x2*)rowp + g;
        const u32x2 v = NTL ? __builtin_nontemporal_load(a) : *a;
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xFFFF0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
}

// Calls f(i0, x[4]) for the 4-token groups g0 + u * NT + t (u < U) of a row,
// t = threadIdx.x; tokens at or past V read as -inf.  All U loads are issued
// before any is used.  Every lane calls f U times, so f may use wave-wide
// operations.  NTL marks the loads non-temporal.
template <int DT, bool NTL, int NT, int U, class F>
__device__ __forceinline__ void load_groups(const Params& p, const void* rowp, uint32_t g0, F&& f)
{
    const uint32_t V = (uint32_t)p.V;
    const uint32_t nfull = V >> 2;
    const uint32_t t = threadIdx.x;
    float x[U][4];
    if (p.vec_in && nfull > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t g = g0 + (uint32_t)u * NT + t;
            load_group<DT, NTL>(rowp, g < nfull ? g : nfull - 1, x[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t g = g0 + (uint32_t)u * NT + t;
            if (g >= nfull) {  // the row's partial last group, or past the row
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t i = 4 * g + j;
                    x[u][j] = i < V ? (DT == kF32 ? ((const float*)rowp)[i]
                                                  : bf16_to_float(((const uint16_t*)rowp)[i]))
                                    : -INFINITY;
                }
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) load4<DT>(rowp, (int64_t)(g0 + (uint32_t)u * NT + t) << 2, V, 0, x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) f((g0 + (uint32_t)u * NT + t) << 2, x[u]);
}

// load_groups over the whole row, kRowUnroll groups per thread per step.
template <int DT, bool NTL, int NT, class F>
__device__ __forceinline__ void stream_row(const Params& p, const void* rowp, F&& f)
{
    const uint32_t ng = ((uint32_t)p.V + 3) >> 2;
    for (uint32_t g0 = 0; g0 < ng; g0 += kRowUnroll * NT) load_groups<DT, NTL, NT, kRowUnroll>(p, rowp, g0, f);
}

// Appends (key, idx) for the lanes with pred to an LDS list: one LDS atomic
// per wave, positions from the lane's rank among the appending lanes.
// Appends past `cap` are counted but dropped.
__device__ __forceinline__ void lds_append(uint32_t* counter, u32x2v* list, uint32_t cap, bool pred, uint32_t key,
                                           uint32_t idx)
{
    const uint64_t mask = __ballot(pred);
    if (mask == 0) return;
    const int leader = __builtin_ctzll(mask);
    const uint32_t lo = (uint32_t)mask, hi = (uint32_t)(mask >> 32);
    uint32_t base = 0;
    if ((int)__lane_id() == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
    if (pred) {
        const uint32_t off = base + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
        if (off < cap) {
            u32x2v e;
            e.x = key;
            e.y = idx;
            list[off] = e;
        }
    }
}

// Per-wave ring of 4-token groups holding at least one kept token: the race
// runs on full waves of such groups instead of on every group of the row.
struct RaceQueue {
    uint32_t i0[kRaceQueue];
    f32x4 x[kRaceQueue];
};


// Per-wave compaction of race work.  A group whose lanes hold a kept token
// joins the wave's ring; once 64 wait, every lane races one.  `race(active,
// i0, x)` is called by all lanes of the wave (it may use wave operations).
template <class Race>
__device__ __forceinline__ void wq_drain(RaceQueue& rq, uint32_t& qh, uint32_t& qn, uint32_t lane, uint32_t cnt,
                                         Race&& race)
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const uint32_t slot = (qh + lane) & (kRaceQueue - 1);
    const f32x4 v = rq.x[slot];
    const float xs[4] = {v.x, v.y, v.z, v.w};
    race(lane < cnt, rq.i0[slot], xs);
    qh = (qh + cnt) & (kRaceQueue - 1);
    qn -= cnt;
}

template <class Race>
__device__ __forceinline__ void wq_push(RaceQueue& rq, uint32_t& qh, uint32_t& qn, uint32_t lane, bool any,
                                        uint32_t i0, const float* xs, Race&& race)
{
    const uint64_t m = __ballot(any);
    if (!m) return;
    if (any) {
        const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint32_t slot = (qh + qn + r) & (kRaceQueue - 1);
        f32x4 v;
        v.x = xs[0]; v.y = xs[1]; v.z = xs[2]; v.w = xs[3];
        rq.i0[slot] = i0;
        rq.x[slot] = v;
    }
    qn += (uint32_t)__popcll(m);
    if (qn >= (uint32_t)kWave) wq_drain(rq, qh, qn, lane, kWave, race);
}

// One race step for a queued group: screen against the best score any wave
// of the workgroup has reached (a score some token achieved, so the screen
// never drops a possible winner), race, and publish the wave's best.
__device__ __forceinline__ void race_queued(const Params& p, int64_t b, bool scored, const RowModel& r,
                                            float c_log2e, float keep_lo, bool active, uint32_t i0, const float* xs,
                                            RaceAcc& acc, float& sstar, uint32_t* shared_bits)
{
    const float shared_best = __uint_as_float(*shared_bits);
    sstar = fmaxf(sstar, shared_best);
    if (active) {
        bool keep[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) keep[j] = xs[j] >= keep_lo;
        race_group(p, b, scored, r, c_log2e, i0, xs, keep, acc, sstar);
    }
    // Publish only when some lane improved on the shared best (after the first
    // few groups that is rare, and the wave reduction is skipped).
    if (__ballot(sstar > shared_best)) {
        const float wave_best = wave_reduce(sstar, MaxF());
        if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(shared_bits, __float_as_uint(wave_best));
    }
}

// Appends (key, idx) for the lanes with pred to a row's list in global memory
// (device-coherent stores): one atomic per wave on the row's counter.
// Appends past `cap` are counted but dropped.
__device__ __forceinline__ void global_append(uint32_t* counter, __amdgpu_buffer_rsrc_t list, uint32_t cap, bool pred,
                                              uint32_t key, uint32_t idx)
{
    const uint64_t mask = __ballot(pred);
    if (mask == 0) return;
    const int leader = __builtin_ctzll(mask);
    uint32_t base = 0;
    if ((int)__lane_id() == leader)
        base = __hip_atomic_fetch_add(counter, (uint32_t)__popcll(mask), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
    if (pred) {
        const uint32_t off = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (off < cap) {
            u32x2v e;
            e.x = key;
            e.y = idx;
            __builtin_amdgcn_raw_buffer_store_b64(e, list, off * 8, 0, kSC1);
        }
    }
}

struct RowShared {
    union {
        struct {
            uint64_t hm[kBins];
            uint32_t hc[kBins];
        } h;
        float factor[kBins];
    } u;
    u32x2v cand[kRowCand];
    RaceQueue rq[kRowThreads / kWave];
    ResolveShared rs;
    double red[64];
    float redf[kMaxWaves], redf2[kMaxWaves];
    int redi[kMaxWaves];
    uint32_t cand_n;
    uint32_t sstar_bits;  // best exact race score found so far in the workgroup (bits of a float >= 0)
};

// Row max, smallest finite logit and error flag over the workgroup: wave
// reductions, then one exchange through LDS.
template <int NT>
__device__ __forceinline__ void block_extremes(float& mx, float& mn, int& bad, float* rf, float* rf2, int* ri)
{
    constexpr int W = NT / kWave;
    mx = wave_reduce(mx, MaxF());
    mn = wave_reduce(mn, MinF());
    bad = wave_reduce(bad, OrI32());
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) {
        rf[w] = mx;
        rf2[w] = mn;
        ri[w] = bad;
    }
    __syncthreads();
    mx = rf[0];
    mn = rf2[0];
    bad = ri[0];
#pragma unroll
    for (int i = 1; i < W; ++i) {
        mx = fmaxf(mx, rf[i]);
        mn = fminf(mn, rf2[i]);
        bad |= ri[i];
    }
}

// Writes the probabilities of tokens i0..i0+3 (those below V), as one
// 16-byte store when the row allows it.
__device__ __forceinline__ void store_probs(float* prow, uint32_t i0, uint32_t V, const float q[4])
{
    if (i0 + 4 <= V && ((uintptr_t)(prow + i0) & 15) == 0) {
        f32x4 v;
        v.x = q[0]; v.y = q[1]; v.z = q[2]; v.w = q[3];
        __builtin_nontemporal_store(v, (f32x4*)(prow + i0));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i0 + j < V) prow[i0 + j] = q[j];
    }
}

// Publishes a row's decided state for race_kernel / probs_kernel and resets
// its race accumulators (plain stores: the next launch on the stream reads them).
static_assert(sizeof(RowModel) <= sizeof(((RowPathState*)nullptr)->model), "RowModel fits its slot");

__device__ __forceinline__ void publish_row(RowPathState* ps, const RowState& st, const RowModel& model, float keep_lo,
                                            float cand_lo)
{
    *(RowModel*)ps->model = model;
    ps->mode = st.mode;
    ps->m = st.m;
    ps->xmin = st.xmin;
    ps->cbin = st.cbin;
    ps->tc = st.tc;
    ps->a_above = st.a_above;
    ps->s_total = st.s_total;
    ps->keep_lo = keep_lo;
    ps->cand_lo = cand_lo;
    ps->best = 0;
    ps->count = 0;
    ps->minkey = 0xFFFFFFFFu;
    ps->cand_n = 0;
    ps->done = 0;
}

// One workgroup of kRowThreads per row.  PUBLISH = false: the whole row
// (passes 1-2, race + candidates, resolver, optional probabilities);
// PUBLISH = true: passes 1-2, then the row's state goes to rw for race_kernel.
template <int DT, bool PUBLISH>
__global__ __launch_bounds__(kRowThreads, 1) void row_kernel(Params p, RowWork rw)
{
    __shared__ RowShared sh;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    const bool want_probs = p.out_probs != nullptr;

    // ---- pass 1: row max, smallest finite logit, NaN / +inf
    float lmax = -INFINITY, lmin = INFINITY;
    int bad = 0;
    stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t, const float* xs) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = xs[j];
            bad |= (v != v) | (v == INFINITY);
            lmax = fmaxf(lmax, v);
            lmin = (v > -INFINITY) ? fminf(lmin, v) : lmin;
        }
    });
    block_extremes<kRowThreads>(lmax, lmin, bad, sh.redf, sh.redf2, sh.redi);
    const RowParams rp = row_params(p, b);
    RowState st;
    st.mode = uniform(first_mode(bad != 0, lmax, rp.T, rp.P, rp.MP, rp.K, want_probs));
    st.m = uniform(lmax);
    st.xmin = uniform(lmin);
    st.cbin = 0;
    st.tc = 0;
    st.a_above = st.s_total = st.s_keep = 0.0;
    RowModel model = {};
    if (st.mode >= kModeTop) model = uniform(make_model(st.m, st.xmin, rp.T, rp.MP));

    // ---- pass 2: bin histogram of the survivors
    if (st.mode == kModeHist) {
        const bool counts = rp.K > 0;
        for (int i = t; i < kBins; i += kRowThreads) {
            sh.u.h.hm[i] = 0;
            sh.u.h.hc[i] = 0;
        }
        __syncthreads();
        // The last bin takes the whole tail of the row: it is summed in
        // registers and added once per wave instead of by LDS atomics.
        uint64_t tail_w = 0;
        uint32_t tail_c = 0;
        stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t, const float* xs) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (survives(model, xs[j])) {
                    const float tp = bin_pos(model, xs[j]);
                    const uint32_t jb = bin_of(tp);
                    const uint32_t fx = bin_fx(model, tp);
                    if (jb == (uint32_t)(kBins - 1)) {
                        tail_w += fx;
                        tail_c += 1;
                    } else {
                        atomicAdd((unsigned long long*)&sh.u.h.hm[jb], (unsigned long long)fx);
                        if (counts) atomicAdd(&sh.u.h.hc[jb], 1u);
                    }
                }
            }
        });
        tail_w = wave_reduce(tail_w, SumU64());
        tail_c = wave_reduce(tail_c, SumU32());
        if ((t & (kWave - 1)) == 0 && tail_c) {
            atomicAdd((unsigned long long*)&sh.u.h.hm[kBins - 1], (unsigned long long)tail_w);
            if (counts) atomicAdd(&sh.u.h.hc[kBins - 1], tail_c);
        }
        __syncthreads();
        const Decision d = decide(model, sh.u.h.hm, counts ? sh.u.h.hc : nullptr, rp.K, rp.P, sh.red);
        st.mode = uniform(d.mode);
        st.cbin = uniform(d.cbin);
        st.tc = uniform(d.tc);
        st.a_above = uniform(d.a_above);
        st.s_total = uniform(d.s_total);
    }

    const Classes cl = classify(model, st);
    const float keep_lo = cl.keep_lo, cand_lo = cl.cand_lo;
    if (PUBLISH) {
        if (t == 0) {
            publish_row(rw.st + b, st, model, keep_lo, cand_lo);
            if (b == 0) *rw.next = 0;  // race_kernel's work counter (it runs after this launch)
        }
        return;
    }

    // ---- pass 3: race the surely kept tokens; the crossing bin's tokens go to LDS
    const bool scored = st.mode != kModeGreedy;
    const bool has_cand = cand_lo < keep_lo;
    const float c_log2e = model.invT * 1.4426950408889634f;
    if (t == 0) {
        sh.cand_n = 0;
        sh.sstar_bits = 0;
    }
    __syncthreads();
    RaceAcc acc;
    acc.init();
    float sstar = 0.0f;
    RaceQueue& rq = sh.rq[t / kWave];
    const uint32_t lane = (uint32_t)t & (kWave - 1);
    uint32_t qh = 0, qn = 0;  // ring head and fill, the same in every lane of the wave
    auto race = [&](bool active, uint32_t i0, const float* xs) __attribute__((always_inline)) {
        race_queued(p, b, scored, model, c_log2e, keep_lo, active, i0, xs, acc, sstar, &sh.sstar_bits);
    };
    stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
        const bool any = (xs[0] >= keep_lo) | (xs[1] >= keep_lo) | (xs[2] >= keep_lo) | (xs[3] >= keep_lo);
        wq_push(rq, qh, qn, lane, any, i0, xs, race);
        if (has_cand) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_append(&sh.cand_n, sh.cand, kRowCand, xs[j] >= cand_lo && xs[j] < keep_lo, order_key(xs[j]),
                           i0 + j);
        }
    });
    if (qn) wq_drain(rq, qh, qn, lane, qn, race);
    acc = block_race<kRowThreads>(acc, sh.rs);
    const uint32_t n = uniform(sh.cand_n);
    if (n <= (uint32_t)kRowCand) {
        resolve_row<kRowThreads>(p, b, model, rp, st, acc,
                                 [&](auto&& fn) {
                                     for (uint32_t i = t; i < n; i += kRowThreads) {
                                         const u32x2v c = sh.cand[i];
                                         fn(c.x, c.y);
                                     }
                                 },
                                 sh.rs);
    } else {  // more candidates than LDS holds: visit the row in global memory
        resolve_row<kRowThreads>(p, b, model, rp, st, acc,
                                 [&](auto&& fn) {
                                     stream_row<DT, false, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
#pragma unroll
                                         for (int j = 0; j < 4; ++j)
                                             if (xs[j] >= cand_lo && xs[j] < keep_lo) fn(order_key(xs[j]), i0 + j);
                                     });
                                 },
                                 sh.rs);
    }
    write_outputs(p, b, st);
    if (!want_probs) return;

    // ---- pass 4: renormalised probabilities
    if (st.mode != kModeError && st.mode != kModeGreedy) prob_factors<kRowThreads>(model, st, sh.u.factor);
    float* prow = p.out_probs + b * p.V;
    const uint32_t V = (uint32_t)p.V;
    stream_row<DT, true, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
        float q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = prob_of(st.mode, model, st, sh.u.factor, xs[j], i0 + j);
        store_probs(prow, i0, V, q);
    });
}

// The chunk a race_kernel / probs_kernel workgroup covers.  Dispatch is
// chunk-major (chunk c of every row, then chunk c + 1), so the workgroups
// resident at any time mix rows that keep many tokens (Philox-bound) with
// rows that keep few (load-bound).  With the row count padded to a multiple
// of 8, all chunks of a row land on one XCD lane (blockIdx mod 8 = row mod 8).
struct ChunkId {
    int64_t b;
    uint32_t chunk;
};
__device__ __forceinline__ ChunkId chunk_id(uint32_t rows_padded)
{
    ChunkId c;
    c.chunk = blockIdx.x / rows_padded;
    c.b = blockIdx.x % rows_padded;
    return c;
}

// The decided part of a row's state, as published by row_kernel.
__device__ __forceinline__ RowState published_state(const RowPathState* ps)
{
    RowState st;
    st.mode = uniform(ps->mode);
    st.m = uniform(ps->m);
    st.xmin = uniform(ps->xmin);
    st.cbin = uniform(ps->cbin);
    st.tc = uniform(ps->tc);
    st.a_above = uniform(ps->a_above);
    st.s_total = uniform(ps->s_total);
    st.s_keep = 0.0;
    st.token = 0;
    st.count = 0;
    st.cut_key = 0;
    return st;
}

struct RaceShared {
    union {
        RaceQueue rq[kRaceThreads / kWave];
        u32x2v cand[kCandLds];  // the resolver's staged candidates
    } u;
    ResolveShared rs;
    uint32_t sstar_bits;
    uint32_t last;
    uint32_t grab[2];  // work items, by iteration parity (see race_kernel)
    uint64_t part_best;
    uint32_t part_count, part_min, part_n;
};

// A row's state as race_kernel needs it.
struct RaceRow {
    RowState st;
    RowModel model;
    RowParams rp;
    float keep_lo, cand_lo, c_log2e;
    bool scored, has_cand;
};

__device__ __forceinline__ RaceRow race_row(const Params& p, const RowPathState* ps, int64_t b)
{
    RaceRow r;
    r.st = published_state(ps);
    r.model = uniform(*(const RowModel*)ps->model);
    r.rp = row_params(p, b);
    r.keep_lo = uniform(ps->keep_lo);
    r.cand_lo = uniform(ps->cand_lo);
    r.scored = r.st.mode != kModeGreedy;
    r.has_cand = r.cand_lo < r.keep_lo;
    r.c_log2e = r.model.invT * 1.4426950408889634f;
    return r;
}

// The last chunks of row b are done: resolve the cut from the merged race
// partial and the row's candidate list, write the outputs.
template <int DT>
__device__ __forceinline__ void resolve_last(const Params& p, const RowWork& rw, int64_t b, RaceRow& r,
                                             RaceShared& sh)
{
    const int t = threadIdx.x;
    RowPathState* ps = rw.st + b;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    const __amdgpu_buffer_rsrc_t rk = coherent(rw.cand + b * kCap);
    if (t == 0) {
        sh.part_best = get(&ps->best);
        sh.part_count = get(&ps->count);
        sh.part_min = get(&ps->minkey);
        sh.part_n = get(&ps->cand_n);
    }
    __syncthreads();
    RaceAcc part;
    part.best = uniform(sh.part_best);
    part.count = uniform(sh.part_count);
    part.minkey = uniform(sh.part_min);
    const uint32_t n = uniform(sh.part_n);
    const float cand_lo = r.cand_lo, keep_lo = r.keep_lo;
    if (n <= (uint32_t)kCandLds) {
        for (uint32_t i0 = t; i0 < n; i0 += 4 * kRaceThreads) {
            u32x2v c[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = i0 + u * kRaceThreads;
                c[u] = __builtin_amdgcn_raw_buffer_load_b64(rk, (i < n ? i : 0) * 8, 0, kSC1);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + u * kRaceThreads < n) sh.u.cand[i0 + u * kRaceThreads] = c[u];
        }
        __syncthreads();
        resolve_row<kRaceThreads>(p, b, r.model, r.rp, r.st, part,
                                  [&](auto&& fn) {
                                      for (uint32_t i = t; i < n; i += kRaceThreads) {
                                          const u32x2v c = sh.u.cand[i];
                                          fn(c.x, c.y);
                                      }
                                  },
                                  sh.rs);
    } else if (n <= (uint32_t)kCap) {
        resolve_row<kRaceThreads>(p, b, r.model, r.rp, r.st, part,
                                  [&](auto&& fn) {
                                      for (uint32_t i = t; i < n; i += kRaceThreads) {
                                          const u32x2v c = __builtin_amdgcn_raw_buffer_load_b64(rk, i * 8, 0, kSC1);
                                          fn(c.x, c.y);
                                      }
                                  },
                                  sh.rs);
    } else {  // the crossing bin overflowed the list: visit the row in global memory
        resolve_row<kRaceThreads>(p, b, r.model, r.rp, r.st, part,
                                  [&](auto&& fn) {
                                      stream_row<DT, false, kRaceThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
#pragma unroll
                                          for (int j = 0; j < 4; ++j)
                                              if (xs[j] >= cand_lo && xs[j] < keep_lo) fn(order_key(xs[j]), i0 + j);
                                      });
                                  },
                                  sh.rs);
    }
    write_outputs(p, b, r.st);
    if (t == 0) {
        ps->token = r.st.token;
        ps->out_count = r.st.count;
        ps->cut_key = r.st.cut_key;
        ps->s_keep = r.st.s_keep;
    }
    __syncthreads();  // the LDS staging area is the race queue's
}

// The race pass, spread over the device: about one resident round of
// workgroups takes 8192-token chunks (row-major) from a counter in the
// workspace, the next one requested while the current one is raced.  A
// workgroup keeps a row's state and race partial across consecutive chunks
// of that row and merges them into the row once per run; the run that
// finishes a row resolves it on the spot.  No workgroup waits for another.
template <int DT>
__global__ __launch_bounds__(kRaceThreads, 4) void race_kernel(Params p, RowWork rw)
{
    __shared__ RaceShared sh;
    const uint32_t N = (uint32_t)rw.N;
    const uint32_t total = (uint32_t)p.B * N;
    const int t = threadIdx.x;
    const uint32_t lane = (uint32_t)t & (kWave - 1);
    const int64_t esz = DT == kF32 ? 4 : 2;
    RaceQueue& rq = sh.u.rq[t / kWave];

    if (t == 0) sh.grab[0] = __hip_atomic_fetch_add(rw.next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    uint32_t item = uniform(sh.grab[0]);
    uint32_t parity = 0;
    int64_t cur = -1;   // row of the current run
    uint32_t run = 0;   // chunks of that row raced since the last merge
    RaceRow r = {};
    RaceAcc acc;
    acc.init();
    float sstar = 0.0f;
    uint32_t qh = 0, qn = 0;
    for (;;) {
        const int64_t b = item < total ? (int64_t)(item / N) : -1;  // -1: no work left
        // A new row, or no work left (possibly on the first grab, when other
        // workgroups took every item first: then there is no run to close).
        if (b != cur || b < 0) {
            if (cur >= 0) {
                // Close the run: drain the queue, merge, and resolve the row if
                // this run finished it.
                RowPathState* pc = rw.st + cur;
                auto race = [&](bool active, uint32_t i0, const float* xs) __attribute__((always_inline)) {
                    race_queued(p, cur, r.scored, r.model, r.c_log2e, r.keep_lo, active, i0, xs, acc, sstar,
                                &sh.sstar_bits);
                };
                if (qn) wq_drain(rq, qh, qn, lane, qn, race);
                acc = block_race<kRaceThreads>(acc, sh.rs);
                if (t == 0 && acc.count) {
                    __hip_atomic_fetch_max(&pc->best, acc.best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_fetch_add(&pc->count, acc.count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_fetch_min(&pc->minkey, acc.minkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                // Every store and atomic of the run completes before it is
                // counted; the run that completes the row then sees them all.
                drain_and_sync();
                if (t == 0)
                    sh.last = (__hip_atomic_fetch_add(&pc->done, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) +
                               run == N);
                __syncthreads();
                if (sh.last) resolve_last<DT>(p, rw, cur, r, sh);
            }
            if (b < 0) break;
            cur = b;
            run = 0;
            acc.init();
            sstar = 0.0f;
            qh = qn = 0;
            r = race_row(p, rw.st + b, b);
            // The screen starts from the best score the row has reached so far.
            if (t == 0) sh.sstar_bits = r.scored ? (uint32_t)(get(&rw.st[b].best) >> 32) : 0u;
            __syncthreads();
        }
        // Ask for the next item now; it is needed only after this chunk.
        uint32_t nxt = 0;
        if (t == 0) nxt = __hip_atomic_fetch_add(rw.next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (r.st.mode != kModeError) {
            const void* rowp = (const char*)p.logits + b * p.stride * esz;
            RowPathState* ps = rw.st + b;
            const __amdgpu_buffer_rsrc_t rk = coherent(rw.cand + b * kCap);
            auto race = [&](bool active, uint32_t i0, const float* xs) __attribute__((always_inline)) {
                race_queued(p, b, r.scored, r.model, r.c_log2e, r.keep_lo, active, i0, xs, acc, sstar,
                            &sh.sstar_bits);
            };
            const float keep_lo = r.keep_lo, cand_lo = r.cand_lo;
            const bool has_cand = r.has_cand;
            load_groups<DT, false, kRaceThreads, kRaceUnroll>(
                p, rowp, (item % N) * (uint32_t)(kRaceChunk / 4), [&](uint32_t i0, const float* xs) {
                    const bool any = (xs[0] >= keep_lo) | (xs[1] >= keep_lo) | (xs[2] >= keep_lo) | (xs[3] >= keep_lo);
                    wq_push(rq, qh, qn, lane, any, i0, xs, race);
                    if (has_cand) {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            global_append(&ps->cand_n, rk, kCap, xs[j] >= cand_lo && xs[j] < keep_lo,
                                          order_key(xs[j]), i0 + j);
                    }
                });
        }
        ++run;
        // A chunk has no workgroup barrier, so thread 0 may publish the next
        // item while a slower wave has yet to read this one: the two live
        // items use alternate slots, and a slot is rewritten only after the
        // barrier every wave passes once it has read it.
        parity ^= 1u;
        if (t == 0) sh.grab[parity] = nxt;
        __syncthreads();
        item = uniform(sh.grab[parity]);
    }
}

// The probability pass of one chunk, after race_kernel has resolved the row.
template <int DT>
__global__ __launch_bounds__(kRaceThreads) void probs_kernel(Params p, RowWork rw)
{
    __shared__ float factor[kBins];
    const ChunkId cid = chunk_id((uint32_t)padded_rows(p.B));
    const int64_t b = cid.b;
    if (b >= p.B) return;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    const RowPathState* ps = rw.st + b;
    RowState st = published_state(ps);
    st.token = uniform(ps->token);
    st.count = uniform(ps->out_count);
    st.cut_key = uniform(ps->cut_key);
    st.s_keep = uniform(ps->s_keep);
    const RowModel model = uniform(*(const RowModel*)ps->model);
    if (st.mode != kModeError && st.mode != kModeGreedy) prob_factors<kRaceThreads>(model, st, factor);
    float* prow = p.out_probs + b * p.V;
    const uint32_t V = (uint32_t)p.V;
    load_groups<DT, true, kRaceThreads, kRaceUnroll>(
        p, rowp, cid.chunk * (uint32_t)(kRaceChunk / 4), [&](uint32_t i0, const float* xs) {
            float q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) q[j] = prob_of(st.mode, model, st, factor, xs[j], i0 + j);
            store_probs(prow, i0, V, q);
        });
}

}  // namespace nucleus
