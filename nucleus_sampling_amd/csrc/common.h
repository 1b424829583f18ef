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
// Wave and workgroup reductions (wave64 shuffles; LDS across waves).
// ---------------------------------------------------------------------------
template <class T, class F>
__device__ __forceinline__ T wave_reduce(T v, F f)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = f(v, __shfl_xor(v, o, kWave));
    return v;
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
    uint64_t x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint64_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
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
