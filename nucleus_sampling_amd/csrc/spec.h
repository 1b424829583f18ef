// spec.h -- speculative-decoding acceptance against the truncated target
// ("Top-p (Nucleus) Sampling, in depth", "Logprobs, speculative decoding and
// reproducibility").  A draft token d, drawn from the draft's own sampling
// distribution q, is accepted with probability min(1, p(d)/q(d)), where p is
// the target's kept, renormalised distribution (nucleus_sample's
// probabilities); otherwise the token is drawn from the normalised positive
// part of p - q.  The result follows p exactly, whatever q is.
//
// Noise: the row's Philox key; counter word 1 = the row index with bit 31
// set, so no word repeats nucleus_sample's race words for the same seed and
// step; words 2-3 = step.  The acceptance uniform u = (r + 1/2) 2^-32 is word
// 0 at counter word 0 = 0xFFFFFFFF (no token reaches it: i / 4 < 2^29); the
// residual draw is the exponential race argmax r_i / E_i over
// r_i = p_i - q_i > 0, token i taking word i mod 4 at counter word 0 = i / 4,
// lowest index on ties.
//
// Two launches.  spec_chunk_kernel: one 256-thread workgroup per 8192-token
// chunk of every row, dispatched chunk-major so a row's chunks spread over
// the device.  Each takes the row's acceptance test (two floats); the chunks
// of a rejected row stream their p and q (8 bytes per token) and race the
// tokens with r_i > 0 behind the same screen as the sampler's race (E >= 1 - u,
// so a token whose 1 - u exceeds r_i / s*, s* the lane's best score so far
// with a margin for rounding, cannot win), and write the chunk's best packed
// score to the caller's workspace.  spec_finish_kernel: one thread per row
// repeats the acceptance test and merges the row's chunk slots in a fixed
// order.  No atomics and no clearing: every slot a merge reads was written
// by this call.
#pragma once

#include "common.h"

namespace nucleus {

constexpr int kSpecThreads = 256;
constexpr int kSpecGroups = 8;                                 // 4-token groups per thread, loads in flight together
constexpr int kSpecChunk = kSpecThreads * kSpecGroups * 4;     // 8192 tokens per workgroup

struct SpecParams {
    const float* target;        // [B, V] kept distribution p
    const float* draft;         // [B, V] draft distribution q
    const int32_t* draft_token; // [B]
    int64_t B, V;
    uint32_t seed_lo, seed_hi, step_lo, step_hi;
    const uint64_t* seeds;      // [B] per-row keys, or null
    int32_t* out_token;         // [B]
    int32_t* out_accepted;      // [B] or null
    uint64_t* part;             // [B][C] chunk results (workspace)
    int C;                      // chunks per row
    int vec;                    // rows 16-byte aligned: 4-token vector loads
};

struct SpecRow {
    uint32_t klo, khi, crow;
    int32_t d;
    bool bad;       // draft token outside [0, V)
    bool accepted;
};

// The row's key and acceptance test: u q(d) < p(d), u from counter word 0 =
// 0xFFFFFFFF.  Pure function of the row's inputs.
__device__ __forceinline__ SpecRow spec_row(const SpecParams& sp, int64_t b)
{
    SpecRow r;
    r.klo = sp.seed_lo;
    r.khi = sp.seed_hi;
    if (sp.seeds) {
        const uint64_t s = sp.seeds[b];
        r.klo = (uint32_t)s;
        r.khi = (uint32_t)(s >> 32);
    }
    r.crow = (uint32_t)b | 0x80000000u;
    r.d = sp.draft_token[b];
    r.bad = r.d < 0 || r.d >= sp.V;
    r.accepted = false;
    if (!r.bad) {
        const float pd = sp.target[b * sp.V + r.d], qd = sp.draft[b * sp.V + r.d];
        // spec_finish_kernel takes one row per lane: the key may differ between lanes.
        const uint4 wu = philox4x32_10_lanes(make_uint4(0xFFFFFFFFu, r.crow, sp.step_lo, sp.step_hi), r.klo, r.khi);
        const double u = ((double)wu.x + 0.5) * 0x1p-32;
        r.accepted = u * (double)qd < (double)pd;
    }
    return r;
}

__global__ __launch_bounds__(kSpecThreads) void spec_chunk_kernel(SpecParams sp)
{
    __shared__ uint64_t red[kSpecThreads / kWave];
    const uint32_t B = (uint32_t)sp.B;
    const int64_t b = blockIdx.x % B;
    const uint32_t c = blockIdx.x / B;
    const uint32_t t = threadIdx.x;
    SpecRow row = spec_row(sp, b);
    row.klo = uniform(row.klo);
    row.khi = uniform(row.khi);
    if (row.bad || row.accepted) return;  // uniform: the whole workgroup leaves; the merge reads no slot

    const uint32_t V = (uint32_t)sp.V;
    const float* P = sp.target + b * sp.V;
    const float* Q = sp.draft + b * sp.V;
    const uint32_t ng = (V + 3) >> 2;
    const uint32_t g0 = c * (kSpecChunk / 4);
    float pv[kSpecGroups][4], qv[kSpecGroups][4];
#pragma unroll
    for (int k = 0; k < kSpecGroups; ++k) {
        const uint32_t g = g0 + (uint32_t)k * kSpecThreads + t;
        if (sp.vec && g < ng) {
            const f32x4 a = __builtin_nontemporal_load((const f32x4*)P + g);
            const f32x4 e = __builtin_nontemporal_load((const f32x4*)Q + g);
            pv[k][0] = a.x; pv[k][1] = a.y; pv[k][2] = a.z; pv[k][3] = a.w;
            qv[k][0] = e.x; qv[k][1] = e.y; qv[k][2] = e.z; qv[k][3] = e.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t i = 4 * g + (uint32_t)j;
                const bool in = g < ng && i < V;
                pv[k][j] = in ? P[in ? i : 0] : 0.0f;
                qv[k][j] = in ? Q[in ? i : 0] : 0.0f;
            }
        }
    }
    uint64_t best = 0;
    float sstar = 0.0f;
#pragma unroll
    for (int k = 0; k < kSpecGroups; ++k) {
        const uint32_t g = g0 + (uint32_t)k * kSpecThreads + t;
        float r[4];
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[j] = pv[k][j] - qv[k][j];
            any |= r[j] > 0.0f;
        }
        if (any) {
            const uint4 w4 = philox4x32_10(make_uint4(g, row.crow, sp.step_lo, sp.step_hi), row.klo, row.khi);
            const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
            // r / sstar * margin; with no score yet every candidate passes.
            const float kk = sstar > 0.0f ? __builtin_amdgcn_rcpf(sstar) * (1.0001f / (1.0f - 1e-4f)) : INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = fmaf((float)(0xFFFFFFFFu - words[j]), 0x1p-32f, 0x1p-33f);  // 1 - u <= E
                if (r[j] > 0.0f && !(w > r[j] * kk)) {
                    const float sc = r[j] / exp1_from_word(words[j]);
                    const uint64_t pk = race_pack(sc, 4 * g + (uint32_t)j);
                    best = pk > best ? pk : best;
                    sstar = fmaxf(sstar, sc);
                }
            }
        }
        // After the first group every lane screens against the wave's best
        // score (a score some token reached, so no possible winner is
        // dropped): with a per-lane bound alone, some lane of the wave would
        // take the exact score at almost every step.
        if (k == 0) sstar = wave_reduce(sstar, MaxF());
    }
    best = block_reduce<kSpecThreads>(best, MaxU64(), red);
    if (t == 0) sp.part[b * sp.C + c] = best;
}

__global__ void spec_finish_kernel(SpecParams sp)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= sp.B) return;
    const SpecRow row = spec_row(sp, b);
    int32_t token = -1, accepted = 0;
    if (!row.bad && row.accepted) {
        token = row.d;
        accepted = 1;
    } else if (!row.bad) {
        uint64_t best = 0;
        for (int c = 0; c < sp.C; ++c) {
            const uint64_t v = sp.part[b * sp.C + c];
            best = v > best ? v : best;
        }
        token = best ? (int32_t)~(uint32_t)best : -1;  // -1: nothing to resample (p is all zero)
    }
    sp.out_token[b] = token;
    if (sp.out_accepted) sp.out_accepted[b] = accepted;
}

}  // namespace nucleus
