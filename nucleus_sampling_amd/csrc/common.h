// common.h -- device building blocks shared by the sampler's kernels (gfx950,
// wave64).  Nothing here allocates; everything is inline device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nucleus {

constexpr int kWave = 64;

// Native clang vectors: the forms the non-temporal load builtins accept.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Order-preserving 32-bit keys of logits.
//
// Ties are numeric equality of the logits ("tied tokens have the same mass
// above them, so they share a fate" -- "Implement batched top-p sampling with
// temperature", "How to approach it"), so the sampler orders tokens by the raw
// logit, never by a rounded x/T: for T > 0 dividing by T preserves the order
// exactly, while rounding x/T to fp32 could merge two distinct logits.
// -0.0 maps to the key of +0.0; bf16 logits are widened exactly first.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float x)
{
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ float bf16_to_float(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

// 2 rej + (a > b): the compare writes VCC and the add takes it as its carry
// in, so a lane's compare results pack into a bit mask at two instructions
// each (false for NaN, as a C compare).
__device__ __forceinline__ uint32_t shift_in_gt(uint32_t rej, float a, float b)
{
    uint32_t r;
    asm("v_cmp_gt_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %3, %3, vcc" : "=v"(r) : "v"(a), "v"(b), "v"(rej) : "vcc");
    return r;
}

// Double to int32, rounding toward zero and saturating at the int32 range
// (NaN gives 0): gfx950's conversion, defined for every input, where a C cast
// of an out-of-range value is not.
__device__ __forceinline__ int32_t cvt_i32_sat(double x)
{
    int32_t r;
    asm("v_cvt_i32_f64 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): per round, words 0 and 2 are multiplied by the two
// round multipliers; the new state is (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the
// key advances by the two Weyl constants between rounds.  philox4x32_10
// needs a wave-uniform key (its schedule lives in scalar registers, and each
// round's two three-way XORs take one instruction each);
// philox4x32_10_lanes takes a key per lane.
// ---------------------------------------------------------------------------

// a ^ b ^ k for a wave-uniform k: gfx950's three-input bitwise operation with
// the truth table of XOR (0x96: set where an odd number of inputs is set).
__device__ __forceinline__ uint32_t xor3_uniform(uint32_t a, uint32_t b, uint32_t k)
{
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
    return r;
}

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1)
{
    // The key schedule is recomputed at every call by scalar adds: left to
    // itself the compiler hoists the twenty round keys out of the callers'
    // loops, runs out of scalar registers and reads them back with one VALU
    // readlane per round key.
    k0 = (uint32_t)__builtin_amdgcn_readfirstlane(k0);  // wave-uniform by contract
    k1 = (uint32_t)__builtin_amdgcn_readfirstlane(k1);
    asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c.z;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c = make_uint4(xor3_uniform(hi1, c.y, k0), lo1, xor3_uniform(hi0, c.w, k1), lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// ---------------------------------------------------------------------------
// The same generator for a key that may differ between lanes (one row per
// lane): plain XORs, no scalar operands.
__device__ __forceinline__ uint4 philox4x32_10_lanes(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c.z;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// Tempered weight e = exp((x - m)/T) in fp32 with the argument carried to
// about one extra word of precision: x - m is split exactly (TwoSum), the
// quotient's remainder is exact by fma, and e^(q + lo) = e^q (1 + lo).  The
// relative error of e is then that of expf alone instead of |a| ulps, which
// keeps race scores well inside a 1e-6 relative margin.
// invT == 0 encodes T = +inf (every finite token weighs 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float tempered_weight(float x, float m, float T, float invT)
{
    const float s = x - m;
    if (s == 0.0f) return 1.0f;
    if (invT == 0.0f) return 1.0f;
    const float q = s * invT;
    const float e = expf(q);
    if (!(e > 0.0f)) return 0.0f;  // underflow, or x - m overflowed to -inf
    const float bb = s - x;
    const float err = (x - (s - bb)) + (-m - bb);  // x - m == s + err exactly
    const float r = fmaf(-q, T, s);                // s - q*T exactly
    const float lo = (r + err) * invT;
    return fmaf(e, lo, e);
}

// Exp(1) variate from a Philox word: u = (r + 1/2)/2^32, E = -ln u, evaluated
// through log1p(-(1-u)) when u >= 1/2 so that small E keeps full relative
// precision.  u and 1-u are formed exactly in double and rounded once.
__device__ __forceinline__ float exp1_from_word(uint32_t r)
{
    if (r < 0x80000000u) {
        const float u = (float)(((double)r + 0.5) * 0x1p-32);
        return -logf(u);
    }
    const uint32_t n = 0xFFFFFFFFu - r;
    const float w = (float)(((double)n + 0.5) * 0x1p-32);
    return -log1pf(-w);
}

// Race score packed for a u64 max: higher score wins, then the lower index.
__device__ __forceinline__ uint64_t race_pack(float score, uint32_t idx)
{
    return ((uint64_t)__float_as_uint(score) << 32) | (uint64_t)(~idx);
}

// ---------------------------------------------------------------------------
// Wave-uniform values (moved to scalar registers).  The argument must be the
// same in every active lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) { return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v))); }
__device__ __forceinline__ uint64_t uniform(uint64_t v)
{
    // readfirstlane returns int: widen through uint32_t so the low word is not
    // sign-extended into the high word.
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ double uniform(double v) { return __longlong_as_double((long long)uniform((uint64_t)__double_as_longlong(v))); }

// ---------------------------------------------------------------------------
// Wave and workgroup reductions and scans.  Inside a wave they move data
// with DPP (a lane reads another lane of its 16-lane row as an operand
// modifier of an ordinary VALU instruction: a few cycles, no LDS round trip)
// and read the four rows' results with v_readlane; across waves through LDS.
// Every lane of the wave must be active.
// ---------------------------------------------------------------------------
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowRor4 = 0x124;   // row_ror:4: lane (l - 4) mod 16 of the row
constexpr int kDppRowRor8 = 0x128;   // row_ror:8
constexpr int kDppRowShr1 = 0x111;   // row_shr:n: lane l - n of the row, 0 below the row's start
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// v of the lane CTRL names (0 bits where it names none), for 4- and 8-byte T.
template <int CTRL, class T>
__device__ __forceinline__ T dpp(T v)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "dpp moves 4- and 8-byte values");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const uint64_t r = ((uint64_t)dpp_u32<CTRL>((uint32_t)(u >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)u);
        return __builtin_bit_cast(T, r);
    }
}

template <class T>
__device__ __forceinline__ T lane_value(T v, int lane)
{
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- and 8-byte values");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, (uint32_t)__builtin_amdgcn_readlane((int)__builtin_bit_cast(uint32_t, v), lane));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    }
}

// f over the 64 lanes (f associative and commutative); every lane receives
// the result, combined in one fixed order.
template <class T, class F>
__device__ __forceinline__ T wave_reduce(T v, F f)
{
    v = f(v, dpp<kDppQuadSwap1>(v));
    v = f(v, dpp<kDppQuadSwap2>(v));  // every lane: its quad
    v = f(v, dpp<kDppRowRor4>(v));    // its quad and the one before
    v = f(v, dpp<kDppRowRor8>(v));    // its row
    return f(f(lane_value(v, 0), lane_value(v, 16)), f(lane_value(v, 32), lane_value(v, 48)));
}

// Inclusive prefix sum over the 64 lanes, in one fixed order: within each
// 16-lane row by doubling steps, then each row adds the rows before it
// ((r0 + r1) + r2 for the last).  Sets `total` to lane 63's value.
template <class T>
__device__ __forceinline__ T wave_inclusive_sum(T v, T& total)
{
    v = v + dpp<kDppRowShr1>(v);
    v = v + dpp<kDppRowShr2>(v);
    v = v + dpp<kDppRowShr4>(v);
    v = v + dpp<kDppRowShr8>(v);
    const T r0 = lane_value(v, 15), r1 = lane_value(v, 31), r2 = lane_value(v, 47);
    const T r01 = r0 + r1, r012 = r01 + r2;
    const int row = (int)(threadIdx.x & (kWave - 1)) >> 4;
    if (row == 1) v = v + r0;
    if (row == 2) v = v + r01;
    if (row == 3) v = v + r012;
    total = lane_value(v, kWave - 1);
    return v;
}

// The inclusive value of the lane before (T(0) for lane 0), given the
// inclusive sums `inc` from wave_inclusive_sum.  Moved as an unsigned bit
// pattern: with the selects written on doubles, the build gave lane 48 the
// wrong value (twice lane 47's), while the same steps on uint64 are exact.
template <class T>
__device__ __forceinline__ T wave_shift_up1(T inc)
{
    using U = std::conditional_t<sizeof(T) == 4, uint32_t, uint64_t>;
    const U u = __builtin_bit_cast(U, inc);
    const U prev = dpp<kDppRowShr1>(u);
    const U r15 = lane_value(u, 15), r31 = lane_value(u, 31), r47 = lane_value(u, 47);
    const int l = (int)(threadIdx.x & (kWave - 1));
    const U r = l == 16 ? r15 : (l == 32 ? r31 : (l == 48 ? r47 : prev));
    return __builtin_bit_cast(T, r);
}

// All threads receive the result.  `scratch` holds one T per wave.
template <int BLOCK, class T, class F>
__device__ __forceinline__ T block_reduce(T v, F f, T* scratch)
{
    constexpr int W = BLOCK / kWave;
    v = wave_reduce(v, f);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) scratch[w] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r = f(r, scratch[i]);
    return r;
}

// Exclusive prefix sum over threads in index order.  `scratch` holds one
// uint64 per wave.
template <int BLOCK>
__device__ __forceinline__ uint64_t block_exclusive_sum(uint64_t v, uint64_t* scratch)
{
    constexpr int W = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    uint64_t wt;
    const uint64_t x = wave_inclusive_sum(v, wt);
    __syncthreads();
    if (lane == kWave - 1) scratch[w] = x;
    __syncthreads();
    uint64_t off = 0;
#pragma unroll
    for (int i = 0; i < W; ++i)
        if (i < w) off += scratch[i];
    return off + x - v;
}

struct MaxU64 { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a > b ? a : b; } };
struct SumU64 { __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; } };
struct MinU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct MaxI32 { __device__ int operator()(int a, int b) const { return a > b ? a : b; } };
struct MinI32 { __device__ int operator()(int a, int b) const { return a < b ? a : b; } };
struct OrI32 { __device__ int operator()(int a, int b) const { return a | b; } };

// ceil(p * S) for p in (0, 1) as an fp32 and S < 2^63, exactly: the integer
// threshold t with  A < p*S  <=>  A < t  for every integer A.
__device__ __forceinline__ uint64_t ceil_p_times(float p, uint64_t S)
{
    const uint32_t bits = __float_as_uint(p);
    const int ex = (int)((bits >> 23) & 0xFF);
    uint32_t mant = bits & 0x7FFFFFu;
    int e2;  // p = mant * 2^e2
    if (ex == 0) { e2 = -149; } else { mant |= 0x800000u; e2 = ex - 150; }
    const unsigned __int128 prod = (unsigned __int128)mant * S;
    const int sh = -e2;  // >= 24 for p < 1
    if (sh >= 128) return prod != 0 ? 1 : 0;
    const unsigned __int128 q = prod >> sh;
    const unsigned __int128 rem = prod - (q << sh);
    return (uint64_t)q + (rem != 0 ? 1 : 0);
}

}  // namespace nucleus
