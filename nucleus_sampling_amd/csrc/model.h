// model.h -- the arithmetic that decides which tokens are kept.
//
// Every path of the sampler (the register-resident split-row kernel, the
// single-workgroup kernel, the last-arriving workgroup's resolver) uses these
// functions and nothing else to weigh tokens, so they all take identical
// decisions, bit for bit.
//
// Weights.  With m the row max and T > 0, token i weighs e_i = exp(-d_i),
// d_i = (m - x_i)/T (the tempered softmax numerator, "What do temperature,
// top-k and top-p each do ...", tempered-softmax equation).
//
// Bins sit on a fixed lattice of the logit that depends on T alone: cell
// a(x) = floor(x s), s = 32/T rounded down to a 24-bit mantissa (so x s is
// exact in double and the cell width in d units is w = 1/(sT), within 2^-23
// of 1/32).  Because the lattice does not move with the row max, a kernel
// can histogram a row in the same pass that finds its max.  With A = a(m),
// a token's bin is j = min(A - a, kBins - 1): bin 0 holds the max, and the
// last bin also takes every token more than ~32 below it (each weighs
// < e^-31.9, so the whole tail moves S by less than V e^-31.9 relative).
//
// Weights are measured from the lattice point (A + 1)/s just above the max:
// token x weighs exp(-(A + 1 - x s) w) = q^j exp(-f w), q = exp(-w),
// f = a + 1 - x s in (0, 1].  That is e_i times one common factor in
// [1, e^w), which every ratio the sampler takes (the top-p threshold, the
// renormalised probabilities) cancels.  The in-bin factor is held as the
// integer
//     fx = floor(2^31 * P(f)),   P = cubic Taylor polynomial of exp(-f w)
// (truncation below 5e-8 relative), so each bin's weight is an exact
// integer sum: associative, hence identical whatever order workgroups or
// lanes add in.
//
// Rules.  A token survives min-p iff x >= max + T ln(min_p) (rounded up to
// fp32; p_i >= min_p * p_max is exactly that inequality).  The cut search
// first locates the crossing bin from bin sums, then resolves the exact cut
// level inside it over integer weights (select.h).  Only bins and the exact
// cut level matter: the bin index is a monotone function of the logit, so
// ties always share a bin and a fate.
#pragma once

#include "common.h"

namespace nucleus {

constexpr int kBins = 1024;
constexpr double kFx = 2147483648.0;  // 2^31

// Row modes decided after the row max is known.
enum : uint32_t {
    kModeError = 1,   // NaN/+inf logit, NaN parameter or no finite logit
    kModeGreedy = 2,  // T <= 0: argmax, lowest index
    kModeTop = 3,     // p <= 0 (and top-k not binding): the top level only
    kModeAll = 4,     // p >= 1 (and top-k not binding): every survivor
    kModeP = 5,       // top-p cut inside one crossing bin
    kModeK = 6,       // top-k binds: every survivor in bins <= the top-k crossing bin is a candidate
    kModeHist = 7,    // (provisional) needs the histogram to decide between the above
};

// The part of the model that depends on T alone: the lattice and the
// in-bin polynomial.
struct Lattice {
    double s;   // cells per logit unit: cell of x = floor(x * s); 0 when T = +inf
    double w;   // cell width in d units, 1/(s T); 0 when every token weighs the same
    double q;   // exp(-w), the weight ratio of neighbouring bin edges
    double q32; // q^32 by five squarings
    float c0, c1, c2, c3;  // 2^31 * Taylor coefficients of exp(-f w)
};

struct RowModel {
    Lattice L;
    double A;      // cell of the row max
    float m;       // row max
    float T;
    float invT;    // 0 for T = +inf
    float tmp;     // min-p threshold: survivor iff x >= tmp; -inf when off
};

// Lattice of temperature T > 0.  Pure function of T.
__device__ __forceinline__ Lattice make_lattice(float T)
{
#pragma clang fp contract(off)
    Lattice L;
    const double sd = 32.0 / (double)T;  // finite for every fp32 T > 0; 0 at +inf
    // Keep 24 significant bits (round toward zero): x * s is then exact.
    L.s = __longlong_as_double(__double_as_longlong(sd) & ~((1ll << 29) - 1));
    const double w = (T == INFINITY) ? 0.0 : 1.0 / (L.s * (double)T);
    L.w = w;
    L.q = exp(-w);
    double q32 = L.q;
#pragma unroll
    for (int k = 0; k < 5; ++k) q32 *= q32;
    L.q32 = q32;
    L.c0 = (float)kFx;
    L.c1 = (float)(-w * kFx);
    L.c2 = (float)(w * w * 0.5 * kFx);
    L.c3 = (float)(-w * w * w * (1.0 / 6.0) * kFx);
    return L;
}

// Cell of a finite logit and its offset f = cell + 1 - x s in (0, 1] (0 only
// past 2^53, where cells are single logits far from any kept token).
__device__ __forceinline__ double lattice_cell(const Lattice& L, float x, float& f)
{
#pragma clang fp contract(off)
    const double pr = (double)x * L.s;  // exact
    const double a = floor(pr);
    f = (float)((a + 1.0) - pr);
    return a;
}

// Integer weight of a token relative to its cell's upper edge, in (0, 2^31].
// The clamp at 0 changes no finite token's weight (the cubic is positive on
// (0, 1]); it gives 0 for f = NaN, which is what -inf yields, so a -inf
// value adds nothing wherever it is binned.
__device__ __forceinline__ uint32_t cell_fx(const Lattice& L, float f)
{
#pragma clang fp contract(off)
    return (uint32_t)fmaxf(fmaf(fmaf(fmaf(L.c3, f, L.c2), f, L.c1), f, L.c0), 0.0f);
}

// Bin of cell a in a row whose max is in cell A.
__device__ __forceinline__ uint32_t bin_of_cell(double A, double a)
{
    const double jd = A - a;
    return jd < (double)(kBins - 1) ? (uint32_t)jd : (uint32_t)(kBins - 1);
}

// Build the model of a row from its max and parameters (T > 0).  Pure
// function of its arguments.
__device__ __forceinline__ RowModel make_model(float m, float T, float mp)
{
#pragma clang fp contract(off)
    RowModel r;
    r.L = make_lattice(T);
    r.A = floor((double)m * r.L.s);
    r.m = m;
    r.T = T;
    r.invT = (T == INFINITY) ? 0.0f : 1.0f / T;
    // min-p: e_i >= mp  <=>  x_i >= m + T ln(mp); at T = +inf every weight is 1.
    float tmp = -INFINITY;
    const float mpc = mp > 1.0f ? 1.0f : mp;
    if (mpc > 0.0f && T != INFINITY) {
        const double t = (double)m + (double)T * log((double)mpc);
        float tf = (float)t;
        if ((double)tf < t) tf = nextafterf(tf, INFINITY);
        tmp = tf;
    }
    r.tmp = tmp;
    return r;
}

// The lattice / model with every field in scalar registers.
__device__ __forceinline__ Lattice uniform(const Lattice& a)
{
    Lattice L;
    L.s = uniform(a.s);
    L.w = uniform(a.w);
    L.q = uniform(a.q);
    L.q32 = uniform(a.q32);
    L.c0 = uniform(a.c0);
    L.c1 = uniform(a.c1);
    L.c2 = uniform(a.c2);
    L.c3 = uniform(a.c3);
    return L;
}

__device__ __forceinline__ RowModel uniform(const RowModel& a)
{
    RowModel r;
    r.L = uniform(a.L);
    r.A = uniform(a.A);
    r.m = uniform(a.m);
    r.T = uniform(a.T);
    r.invT = uniform(a.invT);
    r.tmp = uniform(a.tmp);
    return r;
}

__device__ __forceinline__ bool survives(const RowModel& r, float x)
{
    return x > -INFINITY && x >= r.tmp;
}

// Bin and in-bin integer weight of a finite logit.
struct Binned {
    uint32_t j, fx;
};

__device__ __forceinline__ Binned bin_token(const RowModel& r, float x)
{
    float f;
    const double a = lattice_cell(r.L, x, f);
    Binned o;
    o.j = bin_of_cell(r.A, a);
    o.fx = cell_fx(r.L, f);
    return o;
}

__device__ __forceinline__ uint32_t bin_of(const RowModel& r, float x)
{
    float f;
    return bin_of_cell(r.A, lattice_cell(r.L, x, f));
}

__device__ __forceinline__ uint32_t bin_fx(const RowModel& r, float x)
{
    float f;
    lattice_cell(r.L, x, f);
    return cell_fx(r.L, f);
}

// Weight of bin j's upper edge (0 <= j < 1024), exp(-w)^j as
// q^(j mod 32) * (q^32)^(j / 32) with q = exp(-w): two
// independent five-step binary powerings (a fixed sequence of products, so
// every path computes the same double; relative error below 1e-13).
static_assert(kBins <= 1024, "edge_weight covers ten bits of bin index");
__device__ __forceinline__ double edge_weight(const RowModel& r, int j)
{
#pragma clang fp contract(off)
    double lo = 1.0, hi = 1.0, sl = r.L.q, sh = r.L.q32;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        lo = ((j >> k) & 1) ? lo * sl : lo;
        hi = ((j >> (5 + k)) & 1) ? hi * sh : hi;
        sl *= sl;
        sh *= sh;
    }
    return hi * lo;
}

// Weight of a token at the common 2^-40 scale used when several bins meet
// (the top-k mode): floor(exp(-j w) * fx * 2^9).
__device__ __forceinline__ uint64_t fixed40(const RowModel& r, const Binned& t)
{
#pragma clang fp contract(off)
    return (uint64_t)(edge_weight(r, (int)t.j) * (double)t.fx * 512.0);
}

// Result of reading a full histogram.
struct Decision {
    uint32_t mode;     // kModeP, kModeK, kModeAll or kModeTop
    uint32_t cbin;     // crossing bin (P) or last candidate bin (K)
    uint64_t tc;       // mode P: keep a level of bin cbin iff sum fx above it < tc
    double a_above;    // mode P: weight of bins < cbin
    double s_total;    // weight of all survivors
};

// Weight of bin j: exp(-j w) * H * 2^-31 (0.0 for an empty bin).
__device__ __forceinline__ double bin_weight(const RowModel& r, int j, uint64_t h)
{
#pragma clang fp contract(off)
    return h ? edge_weight(r, j) * ((double)h * (1.0 / kFx)) : 0.0;
}

__device__ __forceinline__ double lane_read_f64(double v, int lane)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Decide how a row's cut is found from its merged histogram H (integer
// weights) and C (counts of survivors per bin, only when k > 0).  H is
// overwritten (with the bin weights, as doubles, transposed).  Must be called by all threads
// of one workgroup.
//
// Deterministic whatever the block size: the weight of bin j is
// exp(-j w) * H[j] * 2^-31, a pure function of j and H[j]; then the first
// wave alone sums them in one fixed order: lane l adds its 16 bins
// 16l .. 16l + 15 one by one from 0.0, a fixed wave scan (wave_inclusive_sum)
// adds the lane totals, and bin j's running weight is (the lanes before l) +
// (its lane's running value).  Counts are integers, exact in any order.  The
// top-p search only stops on non-empty bins, so the cut never lands on an
// empty one whatever the rounding.
__device__ __forceinline__ Decision decide(const RowModel& r, uint64_t* H, uint32_t* C, int k, float p)
{
#pragma clang fp contract(off)
    constexpr int PER = kBins / kWave;  // bins per lane
    __shared__ Decision dec;
    const int t = threadIdx.x;
    // Bin weights, stored transposed over H's space: bin PER l + i (lane l's
    // i-th) at W[i kWave + l], so that the first wave reads them without bank
    // conflicts.  (Blocks of 256 or more threads: four bins a thread at most.)
    double* W = (double*)H;
    double wt[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = t + q * (int)blockDim.x;
        wt[q] = j < kBins ? bin_weight(r, j, H[j]) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = t + q * (int)blockDim.x;
        if (j < kBins) W[(j % PER) * kWave + j / PER] = wt[q];
    }
    __syncthreads();
    if (t < kWave) {
        const int lane = t;
        // The lane's bins in registers, and its total (the searches below
        // redo these sums bin by bin, in the same order, so they see the same
        // values).
        double wv[PER], pre[PER + 1];  // pre[i]: the lane's bins before its i-th, summed in order
        uint32_t crun = 0;
        pre[0] = 0.0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            wv[i] = W[i * kWave + lane];
            pre[i + 1] = pre[i] + wv[i];
            crun += C ? C[PER * lane + i] : 0u;
        }
        const double run = pre[PER];
        // Inclusive wave scans of the lane totals (a fixed order: doubling
        // steps in each 16-lane row, then the rows before), and the
        // inclusive value of the lane before.
        double S;
        uint64_t total;
        const double inc = wave_inclusive_sum(run, S);
        const uint64_t cinc = wave_inclusive_sum((uint64_t)crun, total);
        const double before = wave_shift_up1(inc);
        const uint64_t cbefore = wave_shift_up1(cinc);
        Decision d;
        d.mode = kModeP;
        d.cbin = 0;
        d.tc = 0;
        d.a_above = 0.0;
        d.s_total = S;
        if (C && k > 0 && total > (uint64_t)k) {
            // top-k binds: the first bin where the running count reaches k.
            int first = PER;
            uint32_t cc = 0;
#pragma unroll 4
            for (int i = 0; i < PER; ++i) {
                cc += C[PER * lane + i];
                first = (first == PER && cbefore + cc >= (uint64_t)k) ? i : first;
            }
            const uint64_t m = __ballot(first < PER);
            const int L = m ? (int)__builtin_ctzll(m) : kWave - 1;
            const int i = __builtin_amdgcn_readlane(first < PER ? first : PER - 1, L);
            d.mode = kModeK;
            d.cbin = (uint32_t)(PER * L + i);
        } else if (p >= 1.0f) {
            d.mode = kModeAll;
        } else if (p <= 0.0f) {
            d.mode = kModeTop;
        } else {
            // top-p: the first non-empty bin whose running weight reaches
            // p * S (the last non-empty bin when rounding leaves none).
            // Bin i of the lane has weight before + pre[i] above it and
            // reaches the threshold with before + pre[i + 1]; the tests are
            // independent, so they run side by side.
            const double thr = (double)p * S;
            uint32_t reach = 0, nonempty = 0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const bool ne = wv[i] > 0.0;
                nonempty |= ne ? 1u << i : 0u;
                reach |= (ne && before + pre[i + 1] >= thr) ? 1u << i : 0u;
            }
            const int first = reach ? (int)__builtin_ctz(reach) : PER;
            const int last = nonempty ? 31 - (int)__builtin_clz(nonempty) : -1;
            double above_first = 0.0, above_last = 0.0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const double ab = i > 0 ? before + pre[i] : before;  // weight of the bins before
                above_first = i == first ? ab : above_first;
                above_last = i == last ? ab : above_last;
            }
            const uint64_t mf = __ballot(first < PER);
            int L, i;
            double ab;
            if (mf) {
                L = (int)__builtin_ctzll(mf);
                i = __builtin_amdgcn_readlane(first, L);
                ab = lane_read_f64(above_first, L);
            } else {
                const uint64_t ml = __ballot(last >= 0);  // bin 0 holds the max: never empty
                L = 63 - (int)__builtin_clzll(ml);
                i = __builtin_amdgcn_readlane(last, L);
                ab = lane_read_f64(above_last, L);
            }
            const int j = PER * L + i;
            d.cbin = (uint32_t)j;
            d.a_above = ab;
            // Inside bin j: keep a level iff its fx-sum above < (thr - above) / (e_j 2^-31).
            const double q = (thr - ab) / (edge_weight(r, j) * (1.0 / kFx));
            uint64_t tc = (q <= 1.0) ? 1 : (uint64_t)ceil(q);
            if (!(q < 1.8e19)) tc = ~0ull;
            d.tc = tc;
        }
        if (lane == 0) dec = d;
    }
    __syncthreads();
    const Decision out = dec;
    __syncthreads();
    return out;
}

}  // namespace nucleus
