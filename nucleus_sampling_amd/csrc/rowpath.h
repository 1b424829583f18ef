// rowpath.h -- the sampler's kernels for batches large enough to give every
// row a CU of its own.
//
// row_kernel: one 1024-thread workgroup per row streams the row from global
//   memory once per pass, eight 16-byte loads in flight per thread:
//     1  row max, error flag and, since bins sit on a lattice that does not
//        depend on the max, the bin histogram (LDS)    -> row mode, model,
//                                                         crossing bin (decide)
//     2  only for min-p rows (whose survivors depend on the max), or when
//        the histogram window missed the max: the histogram again
//   then either finishes the row itself (one more pass racing the surely kept
//   tokens and marking the 4-token groups that hold a crossing-bin token,
//   whose tokens are then read again into an LDS list; the resolver; an
//   optional probability pass), or publishes the row's state for
//   race_kernel.
//
// race_kernel: the race pass split into items of 2048 tokens, each raced by
//   one wave on its own, so a row that keeps most of its tokens (whose Philox
//   draws dominate) spreads over many CUs instead of holding one.  Each
//   item merges its race partial into the row's state with order-free
//   atomics (max of the packed score, sums, min) and appends its candidates
//   to the row's list.  No workgroup ever waits for another.
//
// resolve_kernel: one workgroup per row resolves the exact cut from the
//   merged partials and the candidate list, and writes the outputs.
//
// probs_kernel: the optional probability pass, chunked the same way.
//
// Every kernel uses the model's functions and nothing else to weigh tokens,
// so all paths take the same decisions, bit for bit.
#pragma once

#include <type_traits>

#include "prechain.h"
#include "sampler.h"

namespace nucleus {

constexpr int kRowThreads = 1024;  // 16 waves: one workgroup per CU
constexpr int kRowUnroll = 8;      // 4-token groups per thread whose loads are in flight together
// Crossing-bin candidates.  The race pass only marks, in an LDS bitmap, the
// 4-token groups (or runs of 2^k groups in rows of more than 2^18 groups)
// that hold one; after the race the marked groups are listed (up to
// kRowMarked of them), read again and their candidates listed in LDS.
constexpr int kMarkWords = 2048;             // bitmap words: 65536 bits
constexpr int kMarkBits = kMarkWords * 32;
constexpr int kRowMarked = 8192;             // marked groups listed in LDS
constexpr int kRelist = 4;                   // marked groups a thread reads at once
// Min-p rows: the first pass keeps every token within T ln(1/min_p) of the
// max of the first tokens loaded, in per-wave LDS segments of kMinpSeg.
constexpr int kMinpSeg = 256;
constexpr int kMinpCands = kRowMarked / 2;   // their candidates, listed in the marked-group list's space
constexpr int kWin = 4096;         // cells of the fused pass's LDS histogram window
constexpr int kWinHead = kWin - kBins;  // cells the window reaches above the provisional max
constexpr int kRaceQueue = 256;    // per-wave ring of 4-token groups waiting for the race
constexpr int kDrain = 2 * kWave;  // groups raced per drain: two per lane
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

// Loads the 4-token groups g0 + u * NT + t (u < U) of a row into x (t: the
// thread's index among the NT that share the work), all loads issued back to
// back.  fix_groups must run on x before it is used.  NTL marks the loads
// non-temporal.
template <int DT, bool NTL, int NT, int U>
__device__ __forceinline__ void issue_groups(const Params& p, const void* rowp, uint32_t g0, uint32_t t, float x[U][4])
{
    const uint32_t V = (uint32_t)p.V;
    const uint32_t nfull = V >> 2;
    if (p.vec_in && nfull > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t g = g0 + (uint32_t)u * NT + t;
            load_group<DT, NTL>(rowp, g < nfull ? g : nfull - 1, x[u]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) load4<DT>(rowp, (int64_t)(g0 + (uint32_t)u * NT + t) << 2, V, 0, x[u]);
    }
}

// Tokens at or past V read as -inf; the row's partial last group is loaded
// one token at a time.
template <int DT, int NT, int U>
__device__ __forceinline__ void fix_groups(const Params& p, const void* rowp, uint32_t g0, uint32_t t, float x[U][4])
{
    const uint32_t V = (uint32_t)p.V;
    const uint32_t nfull = V >> 2;
    if (!(p.vec_in && nfull > 0)) return;  // the scalar path already did
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t g = g0 + (uint32_t)u * NT + t;
        if (g >= nfull) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t i = 4 * g + j;
                x[u][j] = i < V ? (DT == kF32 ? ((const float*)rowp)[i] : bf16_to_float(((const uint16_t*)rowp)[i]))
                                : -INFINITY;
            }
        }
    }
}

// Calls f(i0, x[4]) for the 4-token groups g0 + u * NT + t (u < U) of a row
// (t: the thread's index among the NT that share the work); tokens at or
// past V read as -inf.  All U loads are issued before any is used.  Every
// lane calls f U times, so f may use wave-wide operations.
template <int DT, bool NTL, int NT, int U, class F>
__device__ __forceinline__ void load_groups(const Params& p, const void* rowp, uint32_t g0, uint32_t t, F&& f)
{
    float x[U][4];
    issue_groups<DT, NTL, NT, U>(p, rowp, g0, t, x);
    fix_groups<DT, NT, U>(p, rowp, g0, t, x);
#pragma unroll
    for (int u = 0; u < U; ++u) f((g0 + (uint32_t)u * NT + t) << 2, x[u]);
}

// Vector loads of the whole groups g0 + u * NT + t (u < U) of an aligned
// row (addresses clamped to the last whole group; mask_whole sets the rest).
template <int DT, bool NTL, int NT, int U>
__device__ __forceinline__ void issue_whole(const void* rowp, uint32_t g0, uint32_t t, uint32_t nfull, float x[U][4])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t g = g0 + (uint32_t)u * NT + t;
        load_group<DT, NTL>(rowp, g < nfull ? g : nfull - 1, x[u]);
    }
}

// Groups past the whole groups read as -inf (selects only: no loads, so the
// loads still in flight for the other buffer are not waited for).
template <int NT, int U>
__device__ __forceinline__ void mask_whole(uint32_t g0, uint32_t t, uint32_t nfull, float x[U][4])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool in = g0 + (uint32_t)u * NT + t < nfull;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[u][j] = in ? x[u][j] : -INFINITY;
    }
}

// Calls f(i0, x[4]) for every 4-token group of the row, the same number of
// times in every lane (so f may use wave-wide operations); a call for no
// token of the row passes -inf values and an i0 past V.  Before the first
// call, every thread calls first(mx) once with the max of the first tokens
// it loaded (-inf if none), so first may use workgroup barriers.
//
// Aligned rows are software-pipelined: two register buffers of
// kRowUnroll / 2 groups per thread, the next one's loads in flight while f
// runs on the current one.  The row's partial last group (V not a multiple
// of 4) takes one more call after the loop, loaded token by token.
template <int DT, bool NTL, int NT, class F, class First, class XF>
__device__ __forceinline__ void stream_row_x(const Params& p, const void* rowp, F&& f, First&& first, XF&& xf)
{
    const uint32_t V = (uint32_t)p.V;
    const uint32_t ng = (V + 3) >> 2, nfull = V >> 2;
    const uint32_t t = threadIdx.x;
    const uint32_t past = ng << 2;  // an i0 no token of the row has
    if (p.vec_in && nfull > 0) {
        constexpr int H = kRowUnroll / 2;
        constexpr uint32_t step = H * NT;
        float xa[H][4], xb[H][4];
        issue_whole<DT, NTL, NT, H>(rowp, 0, t, nfull, xa);
        for (uint32_t g0 = 0; g0 < nfull; g0 += 2 * step) {
            issue_whole<DT, NTL, NT, H>(rowp, g0 + step, t, nfull, xb);
            mask_whole<NT, H>(g0, t, nfull, xa);
#pragma unroll
            for (int u = 0; u < H; ++u) {
                const uint32_t g = g0 + (uint32_t)u * NT + t;
                xf(g < nfull ? g << 2 : past, xa[u]);
            }
            if (g0 == 0) {  // uniform
                float mx = -INFINITY;
#pragma unroll
                for (int u = 0; u < H; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, xa[u][j]);
                first(mx);
            }
#pragma unroll
            for (int u = 0; u < H; ++u) {
                const uint32_t g = g0 + (uint32_t)u * NT + t;
                f(g < nfull ? g << 2 : past, xa[u]);
            }
            if (g0 + step >= nfull) break;  // uniform: the second buffer holds no whole group
            if (g0 + 2 * step < nfull) issue_whole<DT, NTL, NT, H>(rowp, g0 + 2 * step, t, nfull, xa);
            mask_whole<NT, H>(g0 + step, t, nfull, xb);
#pragma unroll
            for (int u = 0; u < H; ++u) {
                const uint32_t g = g0 + step + (uint32_t)u * NT + t;
                xf(g < nfull ? g << 2 : past, xb[u]);
                f(g < nfull ? g << 2 : past, xb[u]);
            }
        }
        if (V & 3u) {  // uniform: the partial last group
            const bool own = t == nfull % NT;
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t i = 4 * nfull + j;
                x[j] = (own && i < V) ? (DT == kF32 ? ((const float*)rowp)[i]
                                                    : bf16_to_float(((const uint16_t*)rowp)[i]))
                                      : -INFINITY;
            }
            xf(own ? nfull << 2 : past, x);
            f(own ? nfull << 2 : past, x);
        }
    } else {  // unaligned rows: token by token
        {
            float x[4];
            load4<DT>(rowp, (int64_t)t << 2, V, 0, x);
            xf(t < ng ? t << 2 : past, x);
            first(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        }
        for (uint32_t g0 = 0; g0 < ng; g0 += NT) {
            const uint32_t g = g0 + t;
            float x[4];
            load4<DT>(rowp, (int64_t)g << 2, V, 0, x);  // -inf past V
            xf(g < ng ? g << 2 : past, x);
            f(g < ng ? g << 2 : past, x);
        }
    }
}

template <int DT, bool NTL, int NT, class F, class First>
__device__ __forceinline__ void stream_row(const Params& p, const void* rowp, F&& f, First&& first)
{
    stream_row_x<DT, NTL, NT>(p, rowp, f, first, [](uint32_t, float*) {});
}

template <int DT, bool NTL, int NT, class F>
__device__ __forceinline__ void stream_row(const Params& p, const void* rowp, F&& f)
{
    stream_row<DT, NTL, NT>(p, rowp, f, [](float) {});
}


// Appends of the crossing-bin tokens of one 4-token group per lane to a
// wave's own LDS area (CAP entries): one wave scan of the lanes' counts gives
// every lane its places, lane by lane in order.  No atomics.  wave_count4
// returns the wave's total and the lane's offset; wave_put4 writes from
// base + offset, dropping entries past CAP (the caller counts them).
template <int N>
__device__ __forceinline__ uint32_t wave_count(const bool c[N], uint32_t& excl)
{
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < N; ++k) cnt += (uint32_t)c[k];
    uint32_t total;
    const uint32_t incl = wave_inclusive_sum(cnt, total);
    excl = incl - cnt;
    return total;
}

__device__ __forceinline__ uint32_t wave_count4(const bool c[4], uint32_t& excl) { return wave_count<4>(c, excl); }

template <uint32_t CAP>
__device__ __forceinline__ void wave_put4(u32x2v* seg, uint32_t off, const bool c[4], const float xs[4], uint32_t i0)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (c[j]) {
            if (off < CAP) {
                u32x2v e;
                e.x = order_key(xs[j]);
                e.y = i0 + (uint32_t)j;
                seg[off] = e;
            }
            ++off;
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
// joins the wave's ring; once kDrain wait, every lane races two (lane l takes
// the l-th and (64 + l)-th oldest).  `race(i0[2], x[2][4], active[2])` is
// called by all lanes of the wave (it may use wave operations).
template <class Race>
__device__ __forceinline__ void wq_drain(RaceQueue& rq, uint32_t& qh, uint32_t& qn, uint32_t lane, uint32_t cnt,
                                         Race&& race)
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint32_t i0[2];
    float xs[2][4];
    bool active[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t k = lane + (uint32_t)h * kWave;
        const uint32_t slot = (qh + k) & (kRaceQueue - 1);
        const f32x4 v = rq.x[slot];
        xs[h][0] = v.x; xs[h][1] = v.y; xs[h][2] = v.z; xs[h][3] = v.w;
        i0[h] = rq.i0[slot];
        active[h] = k < cnt;
    }
    race(i0, xs, active);
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
    if (qn >= (uint32_t)kDrain) wq_drain(rq, qh, qn, lane, kDrain, race);
}

// With no score to screen against yet (a wave's first step), every token
// would pass the screen and be scored one at a time.  Instead every lane
// scores its first kept token (one exact score per lane, all lanes at once)
// and the wave's best of those becomes the bound: a score some token reaches,
// so the screen still keeps every possible winner.
__device__ __forceinline__ void seed_bound(const Params& p, int64_t b, const RowModel& r,
                                                     const uint32_t i0[2], const float xs[2][4],
                                                     const bool keep[2][4], RaceAcc& acc, float& sstar)
{
    int pick = -1;
    float x = 0.0f;
#pragma unroll
    for (int k = 7; k >= 0; --k) {
        const bool kp = keep[k >> 2][k & 3];
        pick = kp ? k : pick;
        x = kp ? xs[k >> 2][k & 3] : x;
    }
    float s = 0.0f;
    if (pick >= 0) {
        const int h = pick >> 2, j = pick & 3;
        const uint32_t gi0 = h ? i0[1] : i0[0];
        const uint4 w4 =
            philox4x32_10(make_uint4(gi0 >> 2, (uint32_t)b, p.step_lo, p.step_hi), p.seed_lo, p.seed_hi);
        s = exact_score(x, r.m, r.T, r.invT, philox_word(w4, (uint32_t)j));
        const uint64_t pk = race_pack(s, gi0 + (uint32_t)j);
        acc.best = pk > acc.best ? pk : acc.best;
    }
    sstar = fmaxf(sstar, wave_reduce(s, MaxF()));
}

// One race step for two queued groups: screen against the best score any
// wave of the workgroup has reached (a score some token achieved, so the
// screen never drops a possible winner), race, and publish the wave's best.
__device__ __forceinline__ void race_queued(const Params& p, int64_t b, bool scored, const RowModel& r,
                                            float c_log2e, float keep_lo, const uint32_t i0[2], const float xs[2][4],
                                            const bool active[2], RaceAcc& acc, float& sstar, uint32_t* shared_bits,
                                            bool track_min)
{
    const float shared_best = __uint_as_float(*shared_bits);
    sstar = fmaxf(sstar, shared_best);
    bool keep[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) keep[h][j] = active[h] && xs[h][j] >= keep_lo;
    if (scored && __ballot(sstar == 0.0f)) seed_bound(p, b, r, i0, xs, keep, acc, sstar);
    race_groups<2>(p, b, scored, r, c_log2e, i0, xs, keep, acc, sstar, track_min);
    // Publish only when some lane improved on the shared best (after the first
    // few groups that is rare, and the wave reduction is skipped).
    if (__ballot(sstar > shared_best)) {
        const float wave_best = wave_reduce(sstar, MaxF());
        if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(shared_bits, __float_as_uint(wave_best));
    }
}

// A wave's staging area for candidates bound for a row's list in global
// memory: appends go to LDS (wave_put4) and are flushed with one atomic
// on the row's counter per kStage entries, instead of one per appending
// group (a returning device atomic stalls the wave for a microsecond).
constexpr int kStage = 256;
static_assert(kStage >= 4 * kWave, "one wave step's candidates fit an emptied stage");

__device__ __forceinline__ void stage_flush(u32x2v* stage, uint32_t& sn, uint32_t* counter,
                                            __amdgpu_buffer_rsrc_t list, uint32_t cap, uint32_t lane)
{
    if (sn == 0) return;
    uint32_t base = 0;
    if (lane == 0) base = __hip_atomic_fetch_add(counter, sn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    for (uint32_t i = lane; i < sn; i += kWave)
        if (base + i < cap) __builtin_amdgcn_raw_buffer_store_b64(stage[i], list, (base + i) * 8, 0, kSC1);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    sn = 0;
}

struct RowShared {
    union {
        struct {  // histogram: a window of lattice cells (bins from decide on)
            uint64_t hm[kWin + kRowThreads];  // the window, then one slot per thread
            uint32_t hc[kWin + kRowThreads];
        } h;
        struct {  // race pass; afterwards the candidate list takes the queues' space
            RaceQueue rq[kRowThreads / kWave];
            uint32_t marks[kMarkWords];       // groups holding a crossing-bin token
            uint32_t marked[kRowMarked];      // the marked groups, listed
        } r;
        float factor[kBins];  // probability pass
    } u;
    ResolveShared rs;
    float redf[kMaxWaves];
    int redi[kMaxWaves];
    uint64_t scan[kMaxWaves];
    uint32_t sstar_bits;  // best exact race score found so far in the workgroup (bits of a float >= 0)
    uint32_t cand_n;      // candidates listed
    uint32_t mcnt[kMaxWaves];  // min-p rows: tokens each wave kept in the first pass
};

// Candidates the LDS list holds after the race (in the race queues' space).
constexpr int kRowCands = (int)(sizeof(RaceQueue) * (kRowThreads / kWave) / sizeof(u32x2v));

struct RowSharedPre : RowShared {
    PreShared pre;
};

static_assert(sizeof(RowShared) <= 160 * 1024 && sizeof(RowSharedPre) <= 160 * 1024, "LDS of one workgroup");
static_assert((kWin + kRowThreads - kBins) * sizeof(uint64_t) >= (size_t)kMinpSeg * (kRowThreads / kWave) * sizeof(u32x2v),
              "min-p segments fit the histogram window past the bins");

// Row max and error flag over the workgroup: wave reductions, then one
// exchange through LDS.
template <int NT>
__device__ __forceinline__ void block_extremes(float& mx, int& bad, float* rf, int* ri)
{
    constexpr int W = NT / kWave;
    mx = wave_reduce(mx, MaxF());
    bad = wave_reduce(bad, OrI32());
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) {
        rf[w] = mx;
        ri[w] = bad;
    }
    __syncthreads();
    mx = rf[0];
    bad = ri[0];
#pragma unroll
    for (int i = 1; i < W; ++i) {
        mx = fmaxf(mx, rf[i]);
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
template <int DT, bool PUBLISH, bool PRE = false>
__global__ __launch_bounds__(kRowThreads, 1) void row_kernel(Params p, RowWork rw)
{
    __shared__ std::conditional_t<PRE, RowSharedPre, RowShared> sh;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    use_row_key(p, b);
    phase_stamp(p, b, kStampStart);
    const bool want_probs = wants_dist(p);  // probabilities or log-probabilities
    // The pre-chain (penalties, grammar mask) is applied to every buffer of
    // every pass as it arrives.
    PreRow pre = {};
    if constexpr (PRE) {
        pre = pre_setup<kRowThreads>(p, b, sh.pre);
    }
    auto xf = [&](uint32_t i0, float* x) __attribute__((always_inline)) {
        if constexpr (PRE) pre_apply(pre, sh.pre, i0, x);
    };
    auto nofirst = [](float) {};

    // ---- pass 1: row max, NaN / +inf; for rows whose
    // need of a histogram the parameters alone decide (no min-p), also the
    // histogram, over a window of lattice cells placed from the max of the
    // first tokens loaded (the lattice does not depend on the max).
    const RowParams rp = row_params(p, b);
    const bool counts = rp.K > 0;
    const bool fused = hist_before_max(rp, want_probs);
    // Min-p rows (their survivors depend on the max, so they cannot bin in
    // the first pass) keep, in per-wave LDS segments past the bins, every
    // token at or above list_lo = (max of the first tokens loaded) + T ln(min_p)
    // rounded down: the survivors are among them, since the row max is at
    // least that first max.  Greedy rows (T <= 0) keep every token at or
    // above that first max: the row max's ties are among them.  When every
    // segment holds its tokens, the histogram and the race pass read the
    // segments instead of the row.
    const bool greedy_row = rp.T <= 0.0f;
    const bool minp_list =
        !PUBLISH && !fused && (greedy_row || (rp.T > 0.0f && rp.T < INFINITY && rp.MP > 0.0f));  // uniform
    float list_lo = INFINITY;  // uniform
    uint32_t mn = 0;           // tokens this wave kept, the same in every lane
    u32x2v* const mseg = (u32x2v*)&sh.u.h.hm[kBins] + (t / kWave) * kMinpSeg;
    const Lattice lat = uniform(make_lattice(fused ? rp.T : 1.0f));
    if (fused)
        for (int i = t; i < kWin + kRowThreads; i += kRowThreads) {
            sh.u.h.hm[i] = 0;
            sh.u.h.hc[i] = 0;
        }
    // lmax takes the IEEE maximum, which propagates NaN, so one test of each
    // thread's max after the pass finds NaN and +inf: no per-token flag.
    float lmax = -INFINITY;
    bool win = false;     // uniform: the window is placed
    double base = 0.0;    // uniform: cell held by window slot 0 (slot k holds cell base - k)
    uint64_t tail_w = 0;  // the second pass: tokens of the last bin, summed in registers
    uint32_t tail_c = 0;
    // The pass, for rows with (COUNTS) and without top-k counts: the test
    // stays out of the per-token code.
    auto pass1 = [&](auto counts_tag) __attribute__((always_inline)) {
        constexpr bool COUNTS = decltype(counts_tag)::value;
        stream_row_x<DT, false, kRowThreads>(
            p, rowp,
            [&](uint32_t i0, const float* xs) {
                lmax = __builtin_elementwise_maximum(
                    lmax, __builtin_elementwise_maximum(__builtin_elementwise_maximum(xs[0], xs[1]),
                                                        __builtin_elementwise_maximum(xs[2], xs[3])));
                if (minp_list) {  // uniform
                    bool c[4];
                    bool any = false;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        c[j] = xs[j] >= list_lo;
                        any |= c[j];
                    }
                    if (__ballot(any)) {  // uniform
                        uint32_t excl;
                        const uint32_t tot = wave_count<4>(c, excl);
                        uint32_t off = mn + excl;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if (c[j]) {
                                if (off < (uint32_t)kMinpSeg) {
                                    u32x2v e;
                                    e.x = __float_as_uint(xs[j]);
                                    e.y = i0 + (uint32_t)j;
                                    mseg[off] = e;
                                }
                                ++off;
                            }
                        }
                        mn += tot;
                    }
                }
                if (win) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // Branch-free.  A token in the window goes to its
                        // cell's slot; every other value goes to this
                        // thread's own slot past the window, which folds
                        // into the last bin: the tail below the window (all
                        // of it in the last bin), a token above the window
                        // (the row is then redone, bins straight from the
                        // model), and NaN / -inf, which are no tokens and add
                        // zero (cell_fx gives them 0; any slot the saturating
                        // conversion picks for them is in range).
                        const float v = xs[j];
                        float f;
                        const double k = base - lattice_cell(lat, v, f);
                        const uint32_t fx = cell_fx(lat, f);
                        const uint32_t ki = (uint32_t)cvt_i32_sat(k);  // k is a whole number
                        const uint32_t slot = ki < (uint32_t)kWin ? ki : (uint32_t)(kWin + t);
                        atomicAdd((unsigned long long*)&sh.u.h.hm[slot], (unsigned long long)fx);
                        if constexpr (COUNTS) atomicAdd(&sh.u.h.hc[slot], v > -INFINITY ? 1u : 0u);
                    }
                }
            },
            [&](float mx) {
                if (!fused && !minp_list) return;
                const float m1 = block_reduce<kRowThreads>(mx, MaxF(), sh.redf);
                if (minp_list) {
                    if (greedy_row) {
                        list_lo = uniform(m1);
                        return;
                    }
                    const float mpc = rp.MP > 1.0f ? 1.0f : rp.MP;
                    const double c = (double)m1 + (double)rp.T * log((double)mpc);
                    float lo = (float)c;
                    if ((double)lo > c) lo = nextafterf(lo, -INFINITY);
                    list_lo = uniform(lo);
                    return;
                }
                base = uniform(floor((double)m1 * lat.s) + (double)kWinHead);
                // Cells are exact integers in double below 2^53; a provisional
                // max of -inf or +inf leaves the window unplaced.
                win = m1 > -INFINITY && fabs(base) < 0x1p50;
            }, xf);
    };
    if (counts) pass1(std::true_type());
    else pass1(std::false_type());
    int bad = !(lmax < INFINITY);  // NaN or +inf
    if (minp_list && (t & (kWave - 1)) == 0) sh.mcnt[t / kWave] = mn;
    block_extremes<kRowThreads>(lmax, bad, sh.redf, sh.redi);  // (its barriers publish mcnt)
    bool use_list = false;  // uniform: the min-p segments hold every token at or above list_lo
    if (minp_list) {
        uint32_t most = 0;
#pragma unroll
        for (int w = 0; w < kRowThreads / kWave; ++w) most = max(most, sh.mcnt[w]);
        use_list = uniform(most) <= (uint32_t)kMinpSeg;
    }
    phase_stamp(p, b, kStampPass1);
    RowState st;
    st.mode = uniform(first_mode(bad != 0, lmax, rp.T, rp.P, rp.MP, rp.K, want_probs));
    st.m = uniform(lmax);
    st.cbin = 0;
    st.tc = 0;
    st.a_above = st.s_total = st.s_keep = 0.0;
    RowModel model = {};
    if (st.mode >= kModeTop) model = uniform(make_model(st.m, rp.T, rp.MP));

    if (st.mode == kModeHist) {
        const int lane = t & (kWave - 1);
        // Bin j of the row is cell A - j: window slot off + j, where
        // off = base - A lies in [0, kWinHead] unless some token rose above
        // the window.  Every slot past off + kBins - 1 and the tail below the
        // window fold into the last bin.
        const double offd = base - model.A;
        uint64_t* H = sh.u.h.hm;
        uint32_t* C = sh.u.h.hc;
        if (win && offd >= 0.0) {
            const uint32_t off = (uint32_t)offd;
            uint64_t fw = 0;
            uint32_t fc = 0;
            for (uint32_t k = off + kBins + t; k < (uint32_t)(kWin + kRowThreads); k += kRowThreads) {
                fw += H[k];
                fc += C[k];
            }
            fw = wave_reduce(fw, SumU64());
            fc = wave_reduce(fc, SumU32());
            if (lane == 0 && (fw || fc)) {
                atomicAdd((unsigned long long*)&H[off + kBins - 1], (unsigned long long)fw);
                if (counts) atomicAdd(&C[off + kBins - 1], fc);
            }
            H += off;
            C += off;
        } else {
            // ---- pass 2 (min-p rows, or the window missed the max): the
            // histogram of the survivors, bins straight from the model.
            for (int i = t; i < kBins; i += kRowThreads) {
                H[i] = 0;
                C[i] = 0;
            }
            __syncthreads();
            // The last bin takes the whole tail of the row: it is summed in
            // registers and added once per wave instead of by LDS atomics.
            tail_w = 0;
            tail_c = 0;
            auto bin_one = [&](float x) __attribute__((always_inline)) {
                if (survives(model, x)) {
                    const Binned bt = bin_token(model, x);
                    if (bt.j == (uint32_t)(kBins - 1)) {
                        tail_w += bt.fx;
                        tail_c += 1;
                    } else {
                        atomicAdd((unsigned long long*)&H[bt.j], (unsigned long long)bt.fx);
                        if (counts) atomicAdd(&C[bt.j], 1u);
                    }
                }
            };
            if (use_list) {  // uniform: every survivor is in the waves' segments
                for (uint32_t i = (uint32_t)lane; i < mn; i += kWave) bin_one(__uint_as_float(mseg[i].x));
            } else {
                stream_row_x<DT, false, kRowThreads>(p, rowp, [&](uint32_t, const float* xs) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) bin_one(xs[j]);
                }, nofirst, xf);
            }
            tail_w = wave_reduce(tail_w, SumU64());
            tail_c = wave_reduce(tail_c, SumU32());
            if (lane == 0 && tail_c) {
                atomicAdd((unsigned long long*)&H[kBins - 1], (unsigned long long)tail_w);
                if (counts) atomicAdd(&C[kBins - 1], tail_c);
            }
        }
        __syncthreads();
        phase_stamp(p, b, kStampHist);
        const Decision d = decide(model, H, counts ? C : nullptr, rp.K, rp.P);
        phase_stamp(p, b, kStampDecide);
        st.mode = uniform(d.mode);
        st.cbin = uniform(d.cbin);
        st.tc = uniform(d.tc);
        st.a_above = uniform(d.a_above);
        st.s_total = uniform(d.s_total);
    }

    const Classes cl = classify(model, st);
    const float keep_lo = cl.keep_lo, cand_lo = cl.cand_lo;
    phase_stamp(p, b, kStampClassify);
    if (PUBLISH) {
        if (t == 0) publish_row(rw.st + b, st, model, keep_lo, cand_lo);
        return;
    }

    const uint32_t V = (uint32_t)p.V;
    if (use_list) {  // uniform
        // ---- pass 3 of a min-p or greedy row from its segments: every kept
        // token and every candidate is there.  Kept tokens are raced one by one; the
        // candidates are placed in one list (one wave scan and one LDS atomic
        // per wave step) in the marked-group list's space, which neither the
        // segments nor the bins use.
        const uint32_t lane = (uint32_t)t & (kWave - 1);
        u32x2v* const clist = (u32x2v*)sh.u.r.marked;
        static_assert(sizeof(sh.u.r.marked) >= sizeof(u32x2v) * kMinpCands, "candidate list fits");
        if (t == 0) sh.cand_n = 0;
        __syncthreads();
        RaceAcc acc;
        acc.init();
        for (uint32_t base = 0; base < mn; base += kWave) {  // uniform in the wave
            const uint32_t i = base + lane;
            bool c = false;
            uint32_t key = 0, idx = 0;
            if (i < mn) {
                const u32x2v e = mseg[i];
                const float x = __uint_as_float(e.x);
                key = order_key(x);
                idx = e.y;
                if (x >= keep_lo) {
                    if (greedy_row) {  // uniform: every kept token scores 1, so the lowest index wins
                        const uint64_t pk = race_pack(1.0f, idx);
                        acc.best = pk > acc.best ? pk : acc.best;
                        acc.count += 1;
                        acc.minkey = key < acc.minkey ? key : acc.minkey;
                    } else {
                        race_one(p, b, model, key, idx, acc);
                    }
                }
                c = x >= cand_lo && x < keep_lo;
            }
            uint32_t tot;
            const uint32_t incl = wave_inclusive_sum((uint32_t)c, tot);
            uint32_t at = 0;
            if (lane == 0 && tot) at = atomicAdd(&sh.cand_n, tot);
            const uint32_t off = (uint32_t)__builtin_amdgcn_readlane((int)at, 0) + incl - (uint32_t)c;
            if (c && off < (uint32_t)kMinpCands) {
                u32x2v e;
                e.x = key;
                e.y = idx;
                clist[off] = e;
            }
        }
        acc = block_race<kRowThreads>(acc, sh.rs);  // (its barriers publish the list)
        phase_stamp(p, b, kStampPass3);
        const uint32_t n = uniform(sh.cand_n);
        phase_fact(p, b, kStampMode, st.mode);
        phase_fact(p, b, kStampCands, n);
        if (n <= (uint32_t)kMinpCands) {
            resolve_row<kRowThreads>(p, b, model, rp, st, acc, cl,
                                     [&](auto&& fn) {
                                         for (uint32_t k = t; k < n; k += kRowThreads) {
                                             const u32x2v e = clist[k];
                                             fn(e.x, e.y);
                                         }
                                     },
                                     sh.rs);
        } else {  // more candidates than the list holds: visit the row in global memory
            resolve_row<kRowThreads>(p, b, model, rp, st, acc, cl,
                                     [&](auto&& fn) {
                                         stream_row_x<DT, false, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
#pragma unroll
                                             for (int j = 0; j < 4; ++j)
                                                 if (xs[j] >= cand_lo && xs[j] < keep_lo) fn(order_key(xs[j]), i0 + j);
                                         }, nofirst, xf);
                                     },
                                     sh.rs);
        }
    } else {
        // ---- pass 3: race the surely kept tokens; mark the groups that hold a
        // crossing-bin token
        const bool scored = st.mode != kModeGreedy;
        const bool has_cand = cand_lo < keep_lo;
        const float c_log2e = model.invT * 1.4426950408889634f;
        const uint32_t ngroups = (V + 3) >> 2;
        // Groups per mark: 1, or the power of two that fits the row in kMarkBits.
        uint32_t mshift = 0;
        while ((ngroups - 1) >> mshift >= (uint32_t)kMarkBits) ++mshift;
        const uint32_t nmarks = ((ngroups - 1) >> mshift) + 1;
        __syncthreads();  // every thread is past decide: the histogram's space is free
        for (uint32_t i = t; i < (uint32_t)kMarkWords; i += kRowThreads) sh.u.r.marks[i] = 0;
        if (t == 0) {
            sh.sstar_bits = 0;
            sh.cand_n = 0;
        }
        __syncthreads();
        RaceAcc acc;
        acc.init();
        float sstar = 0.0f;
        RaceQueue& rq = sh.u.r.rq[t / kWave];
        const uint32_t lane = (uint32_t)t & (kWave - 1);
        uint32_t qh = 0, qn = 0;  // ring head and fill, the same in every lane of the wave
        // A group joins its wave's ring if it holds a surely kept token or a
        // candidate; each drain races the kept tokens of its groups and marks
        // those holding a candidate (one LDS or per such group: in a dense row
        // nearly every drain holds a candidate, and a mark costs far less than
        // placing each candidate in a list).
        const float push_lo = has_cand ? cand_lo : keep_lo;
        auto race = [&](const uint32_t* i0, const float (*xs)[4], const bool* active) __attribute__((always_inline)) {
            race_queued(p, b, scored, model, c_log2e, keep_lo, i0, xs, active, acc, sstar, &sh.sstar_bits, !has_cand);
            if (has_cand) {  // uniform
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bool c = false;
#pragma unroll
                    for (int j = 0; j < 4; ++j) c |= (xs[h][j] >= cand_lo) & (xs[h][j] < keep_lo);
                    if (active[h] && c) {
                        const uint32_t m = (i0[h] >> 2) >> mshift;
                        atomicOr(&sh.u.r.marks[m >> 5], 1u << (m & 31));
                    }
                }
            }
        };
        stream_row_x<DT, false, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
            const bool any = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])) >= push_lo;
            wq_push(rq, qh, qn, lane, any, i0, xs, race);
        }, nofirst, xf);
        if (qn) wq_drain(rq, qh, qn, lane, qn, race);
        acc = block_race<kRowThreads>(acc, sh.rs);  // (its barriers publish the marks)
        phase_stamp(p, b, kStampPass3);

        // The marked groups, listed in order by one scan of the marks' counts.
        uint32_t nmarked = 0;
        if (has_cand) {  // uniform
            constexpr int kWordsPerThread = kMarkWords / kRowThreads;
            uint32_t words[kWordsPerThread];
            uint32_t cnt = 0;
#pragma unroll
            for (int k = 0; k < kWordsPerThread; ++k) {
                const uint32_t wi = (uint32_t)t * kWordsPerThread + k;
                words[k] = wi * 32 < nmarks ? sh.u.r.marks[wi] : 0u;
                cnt += (uint32_t)__builtin_popcount(words[k]);
            }
            uint32_t off = (uint32_t)block_exclusive_sum<kRowThreads>(cnt, sh.scan);
#pragma unroll
            for (int w = 0; w < kRowThreads / kWave; ++w) nmarked += (uint32_t)sh.scan[w];  // the waves' totals
            nmarked = uniform(nmarked);
#pragma unroll
            for (int k = 0; k < kWordsPerThread; ++k) {
                uint32_t w = words[k];
                while (w) {
                    const uint32_t m = ((uint32_t)t * kWordsPerThread + k) * 32 + (uint32_t)__builtin_ctz(w);
                    w &= w - 1u;
                    if (off < (uint32_t)kRowMarked) sh.u.r.marked[off] = m;
                    ++off;
                }
            }
            __syncthreads();
        }
        phase_fact(p, b, kStampMode, st.mode);
        phase_fact(p, b, kStampMarked, nmarked);
        const uint32_t per_mark = 1u << mshift;
        u32x2v* const list = (u32x2v*)sh.u.r.rq;
        bool listed = false;  // uniform: the candidates fit the LDS list
        if (nmarked <= (uint32_t)kRowMarked && nmarked * per_mark <= (uint32_t)(4 * kRowCands)) {
            // Read the marked groups again (kRelist loads in flight per thread) and
            // list their candidates; every lane runs the same number of steps,
            // so the placing may use wave operations.
            const uint32_t total = nmarked * per_mark;
            for (uint32_t base = 0; base < total; base += kRelist * kRowThreads) {
                float x[kRelist][4];
                uint32_t g[kRelist];
#pragma unroll
                for (int u = 0; u < kRelist; ++u) {
                    const uint32_t k = base + (uint32_t)u * kRowThreads + (uint32_t)t;
                    g[u] = k < total ? (sh.u.r.marked[k >> mshift] << mshift) + (k & (per_mark - 1)) : ngroups;
                    load4<DT>(rowp, (int64_t)min(g[u], ngroups) << 2, V, p.vec_in, x[u]);  // -inf past V
                }
                // One wave scan of the lanes' counts and one LDS atomic a wave
                // place the candidates.
                bool c[kRelist][4];
                uint32_t cnt = 0;
#pragma unroll
                for (int u = 0; u < kRelist; ++u) {
                    xf(g[u] << 2, x[u]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        c[u][j] = g[u] < ngroups && x[u][j] >= cand_lo && x[u][j] < keep_lo;
                        cnt += (uint32_t)c[u][j];
                    }
                }
                uint32_t tot;
                const uint32_t incl = wave_inclusive_sum(cnt, tot);
                uint32_t at = 0;
                if (lane == 0 && tot) at = atomicAdd(&sh.cand_n, tot);
                uint32_t off = (uint32_t)__builtin_amdgcn_readlane((int)at, 0) + incl - cnt;
#pragma unroll
                for (int u = 0; u < kRelist; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (c[u][j]) {
                            if (off < (uint32_t)kRowCands) {
                                u32x2v e;
                                e.x = order_key(x[u][j]);
                                e.y = (g[u] << 2) + (uint32_t)j;
                                list[off] = e;
                            }
                            ++off;
                        }
                    }
            }
            __syncthreads();
            const uint32_t n = uniform(sh.cand_n);
            phase_fact(p, b, kStampCands, n);
            if (n <= (uint32_t)kRowCands) {
                resolve_row<kRowThreads>(p, b, model, rp, st, acc, cl,
                                         [&](auto&& fn) {
                                             for (uint32_t i = t; i < n; i += kRowThreads) {
                                                 const u32x2v c = list[i];
                                                 fn(c.x, c.y);
                                             }
                                         },
                                         sh.rs);
                listed = true;
            }
        }
        if (!listed) {  // more candidates than LDS holds: visit the row in global memory
            resolve_row<kRowThreads>(p, b, model, rp, st, acc, cl,
                                     [&](auto&& fn) {
                                         stream_row_x<DT, false, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
#pragma unroll
                                             for (int j = 0; j < 4; ++j)
                                                 if (xs[j] >= cand_lo && xs[j] < keep_lo) fn(order_key(xs[j]), i0 + j);
                                         }, nofirst, xf);
                                     },
                                     sh.rs);
        }
    }
    write_outputs(p, b, st);
    phase_stamp(p, b, kStampResolve);
    if (!want_probs) {
        phase_stamp(p, b, kStampProbs);
        return;
    }

    // ---- pass 4: renormalised probabilities and / or log-probabilities
    if (p.out_probs && st.mode != kModeError && st.mode != kModeGreedy)
        prob_factors<kRowThreads>(model, st, sh.u.factor);
    const LogNorm ln = log_norm(model, st);
    float* prow = p.out_probs ? p.out_probs + b * p.V : nullptr;
    float* lrow = p.out_logprobs ? p.out_logprobs + b * p.V : nullptr;
    stream_row_x<DT, true, kRowThreads>(p, rowp, [&](uint32_t i0, const float* xs) {
        float q[4];
        if (prow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) q[j] = prob_of(st.mode, model, st, sh.u.factor, xs[j], i0 + j);
            store_probs(prow, i0, V, q);
        }
        if (lrow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) q[j] = logprob_of(st.mode, model, st, ln, xs[j], i0 + j);
            store_probs(lrow, i0, V, q);
        }
    }, nofirst, xf);
    phase_stamp(p, b, kStampProbs);
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

// ---------------------------------------------------------------------------
// The chunked race (race_kernel) and the per-row resolver (resolve_kernel).
// ---------------------------------------------------------------------------
constexpr int kItemGroups = 8;                         // groups per lane per work item
constexpr int kItemTokens = kWave * kItemGroups * 4;   // 2048 tokens per item

// Every wave of race_kernel works alone on 2048-token items of the batch:
// item k is chunk c = k / B of row (k + c) % B, and wave w of the W launched
// takes items w, w + W, w + 2W, ...  The waves resident on a CU thus hold
// chunks of many rows, so rows that keep many tokens (whose Philox draws dominate) and rows
// that keep few share every CU.  A wave races its item's kept tokens through
// its ring, appends the item's candidates to the row's list (staged in LDS,
// one atomic on the row's counter per flush) and merges its
// race partial into the row with order-free atomics (max of the packed
// score, sums, min).  No barrier, no waiting, no shared work counter:
// resolve_kernel, the next launch, reads the merged results.
template <int DT>
__global__ __launch_bounds__(kRaceThreads, 4) void race_kernel(Params p, RowWork rw)
{
    __shared__ RaceQueue rings[kRaceThreads / kWave];
    __shared__ u32x2v stages[kRaceThreads / kWave][kStage];
    const uint32_t lane = threadIdx.x & (kWave - 1);
    RaceQueue& rq = rings[threadIdx.x / kWave];
    u32x2v* const stage = stages[threadIdx.x / kWave];
    const uint32_t B = (uint32_t)p.B;
    const uint32_t NI = (uint32_t)rw.N;  // items per row
    const uint32_t total = B * NI;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const uint32_t waves = gridDim.x * (kRaceThreads / kWave);
    // The current item's row and its published state (wave-uniform).
    int64_t b = 0;
    uint32_t g0 = 0;  // the item's first 4-token group
    RowPathState* ps = nullptr;
    RowModel model = {};
    float keep_lo = INFINITY, cand_lo = INFINITY, c_log2e = 0.0f, wbest = 0.0f, sstar = 0.0f;
    bool scored = false, has_cand = false;
    __amdgpu_buffer_rsrc_t rk;
    auto where = [&](uint32_t it, int64_t& rb, uint32_t& rg0) {
        // Chunk c of the rows is rotated by c, so that a wave whose stride is
        // a multiple of B still meets a different row at every item.
        const uint32_t chunk = it / B;
        rb = (int64_t)((it % B + chunk) % B);
        rg0 = chunk * (uint32_t)(kItemTokens / 4);
    };
    auto rowp_of = [&](int64_t rb) { return (const void*)((const char*)p.logits + rb * p.stride * esz); };
    auto open_item = [&](int64_t rb) {
        use_row_key(p, rb);
        ps = rw.st + rb;
        const uint32_t mode = uniform(ps->mode);
        model = uniform(*(const RowModel*)ps->model);
        const bool live = mode != kModeError;  // error rows: no token compares >= NaN
        keep_lo = live ? uniform(ps->keep_lo) : __builtin_nanf("");
        cand_lo = live ? uniform(ps->cand_lo) : __builtin_nanf("");
        scored = mode != kModeGreedy;
        has_cand = cand_lo < keep_lo;
        c_log2e = model.invT * 1.4426950408889634f;
        rk = coherent(rw.cand + rb * kCap);
        // The screen starts from the best score the row has reached so far.
        wbest = (scored && live) ? __uint_as_float((uint32_t)(get(&ps->best) >> 32)) : 0.0f;
        sstar = wbest;
    };

    RaceAcc acc;
    acc.init();
    uint32_t qh = 0, qn = 0;
    uint32_t sn = 0;  // staged candidates, the same in every lane
    auto race = [&](const uint32_t* i0, const float (*xs)[4], const bool* active) __attribute__((always_inline)) {
        bool keep[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) keep[h][j] = active[h] && xs[h][j] >= keep_lo;
        if (scored && __ballot(sstar == 0.0f)) seed_bound(p, b, model, i0, xs, keep, acc, sstar);
        race_groups<2>(p, b, scored, model, c_log2e, i0, xs, keep, acc, sstar, !has_cand);
        // Share the wave's best score only when some lane improved it.
        if (__ballot(sstar > wbest)) wbest = wave_reduce(sstar, MaxF());
        sstar = fmaxf(sstar, wbest);
    };
    auto group = [&](uint32_t i0, const float* xs) {
        const bool any = (xs[0] >= keep_lo) | (xs[1] >= keep_lo) | (xs[2] >= keep_lo) | (xs[3] >= keep_lo);
        wq_push(rq, qh, qn, lane, any, i0, xs, race);
        if (has_cand) {
            bool c[4];
            bool anyc = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = xs[j] >= cand_lo && xs[j] < keep_lo;
                anyc |= c[j];
            }
            if (__ballot(anyc)) {  // uniform: most groups hold no crossing-bin token
                uint32_t excl;
                const uint32_t tot = wave_count4(c, excl);  // at most 4 kWave = kStage
                if (sn + tot > (uint32_t)kStage) stage_flush(stage, sn, &ps->cand_n, rk, kCap, lane);
                wave_put4<kStage>(stage, sn + excl, c, xs, i0);
                sn += tot;
            }
        }
    };
    // End of an item: race what the ring holds, hand the candidates over and
    // merge the race partial into the row.
    auto close_item = [&]() {
        if (qn) wq_drain(rq, qh, qn, lane, qn, race);
        stage_flush(stage, sn, &ps->cand_n, rk, kCap, lane);
        const uint64_t best = wave_reduce(acc.best, MaxU64());
        const uint32_t count = wave_reduce(acc.count, SumU32());
        const uint32_t minkey = wave_reduce(acc.minkey, MinU32());
        if (lane == 0 && count) {
            __hip_atomic_fetch_max(&ps->best, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&ps->count, count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_min(&ps->minkey, minkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        acc.init();
    };

    for (uint32_t item = blockIdx.x * (kRaceThreads / kWave) + threadIdx.x / kWave; item < total; item += waves) {
        where(item, b, g0);
        open_item(b);
        load_groups<DT, false, kWave, kItemGroups>(p, rowp_of(b), g0, lane, group);
        close_item();
    }
}

struct ResolveKShared {
    u32x2v cand[kCandLds];
    ResolveShared rs;
};

// After race_kernel: one workgroup per row resolves the exact cut from the
// merged race partial and the row's candidate list, and writes the outputs.
template <int DT>
__global__ __launch_bounds__(kRowThreads) void resolve_kernel(Params p, RowWork rw)
{
    __shared__ ResolveKShared sh;
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    use_row_key(p, b);
    RowPathState* ps = rw.st + b;
    RowState st = published_state(ps);
    const RowModel model = uniform(*(const RowModel*)ps->model);
    const RowParams rp = row_params(p, b);
    const float cand_lo = uniform(ps->cand_lo), keep_lo = uniform(ps->keep_lo);
    Classes cl;
    cl.keep_lo = keep_lo;
    cl.cand_lo = cand_lo;
    RaceAcc part;
    part.best = uniform(ps->best);
    part.count = uniform(ps->count);
    part.minkey = uniform(ps->minkey);
    const uint32_t n = uniform(ps->cand_n);
    const uint2* list = rw.cand + b * kCap;
    const int64_t esz = DT == kF32 ? 4 : 2;
    const void* rowp = (const char*)p.logits + b * p.stride * esz;
    if (n <= (uint32_t)kCandLds) {
        for (uint32_t i = t; i < n; i += kRowThreads) {
            const uint2 c = list[i];
            u32x2v e;
            e.x = c.x;
            e.y = c.y;
            sh.cand[i] = e;
        }
        __syncthreads();
        resolve_row<kRowThreads>(p, b, model, rp, st, part, cl,
                                  [&](auto&& fn) {
                                      for (uint32_t i = t; i < n; i += kRowThreads) {
                                          const u32x2v c = sh.cand[i];
                                          fn(c.x, c.y);
                                      }
                                  },
                                  sh.rs);
    } else if (n <= (uint32_t)kCap) {
        resolve_row<kRowThreads>(p, b, model, rp, st, part, cl,
                                  [&](auto&& fn) {
                                      for (uint32_t i = t; i < n; i += kRowThreads) {
                                          const uint2 c = list[i];
                                          fn(c.x, c.y);
                                      }
                                  },
                                  sh.rs);
    } else {  // the crossing bin overflowed the list: visit the row in global memory
        resolve_row<kRowThreads>(p, b, model, rp, st, part, cl,
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
    if (t == 0) {
        ps->token = st.token;
        ps->out_count = st.count;
        ps->cut_key = st.cut_key;
        ps->s_keep = st.s_keep;
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
    if (p.out_probs && st.mode != kModeError && st.mode != kModeGreedy) prob_factors<kRaceThreads>(model, st, factor);
    const LogNorm ln = log_norm(model, st);
    float* prow = p.out_probs ? p.out_probs + b * p.V : nullptr;
    float* lrow = p.out_logprobs ? p.out_logprobs + b * p.V : nullptr;
    const uint32_t V = (uint32_t)p.V;
    load_groups<DT, true, kRaceThreads, kRaceUnroll>(
        p, rowp, cid.chunk * (uint32_t)(kRaceChunk / 4), threadIdx.x, [&](uint32_t i0, const float* xs) {
            float q[4];
            if (prow) {
#pragma unroll
                for (int j = 0; j < 4; ++j) q[j] = prob_of(st.mode, model, st, factor, xs[j], i0 + j);
                store_probs(prow, i0, V, q);
            }
            if (lrow) {
#pragma unroll
                for (int j = 0; j < 4; ++j) q[j] = logprob_of(st.mode, model, st, ln, xs[j], i0 + j);
                store_probs(lrow, i0, V, q);
            }
        });
}

}  // namespace nucleus
