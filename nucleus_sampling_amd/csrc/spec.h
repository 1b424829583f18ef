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
// One workgroup per row.  The acceptance test reads two floats; only a
// rejected row streams its p and q rows (8 bytes per token), racing the
// tokens with r_i > 0 behind the same screen as the sampler's race: E >= 1 - u,
// so a token whose 1 - u exceeds r_i / s* (s* the lane's best score so far,
// with a margin for rounding) cannot win.
#pragma once

#include "common.h"

namespace nucleus {

constexpr int kSpecThreads = 512;
constexpr int kSpecUnroll = 4;  // groups of 4 tokens per thread with loads in flight together

struct SpecParams {
    const float* target;        // [B, V] kept distribution p
    const float* draft;         // [B, V] draft distribution q
    const int32_t* draft_token; // [B]
    int64_t B, V;
    uint32_t seed_lo, seed_hi, step_lo, step_hi;
    const uint64_t* seeds;      // [B] per-row keys, or null
    int32_t* out_token;         // [B]
    int32_t* out_accepted;      // [B] or null
    int vec;                    // rows 16-byte aligned: 4-token vector loads
};

__global__ __launch_bounds__(kSpecThreads) void spec_kernel(SpecParams sp)
{
    __shared__ uint64_t red[kSpecThreads / kWave];
    const int64_t b = blockIdx.x;
    const uint32_t t = threadIdx.x;
    uint32_t klo = sp.seed_lo, khi = sp.seed_hi;
    if (sp.seeds) {
        const uint64_t s = sp.seeds[b];
        klo = (uint32_t)s;
        khi = (uint32_t)(s >> 32);
    }
    klo = uniform(klo);
    khi = uniform(khi);
    const uint32_t crow = (uint32_t)b | 0x80000000u;
    const uint32_t V = (uint32_t)sp.V;
    const int32_t d = uniform((uint32_t)sp.draft_token[b]);
    if (d < 0 || (uint32_t)d >= V) {  // uniform: the whole workgroup leaves
        if (t == 0) {
            sp.out_token[b] = -1;
            if (sp.out_accepted) sp.out_accepted[b] = 0;
        }
        return;
    }
    const float* P = sp.target + b * sp.V;
    const float* Q = sp.draft + b * sp.V;
    const float pd = uniform(P[d]), qd = uniform(Q[d]);
    const uint4 wu = philox4x32_10(make_uint4(0xFFFFFFFFu, crow, sp.step_lo, sp.step_hi), klo, khi);
    const double u = ((double)wu.x + 0.5) * 0x1p-32;
    if (u * (double)qd < (double)pd) {  // uniform
        if (t == 0) {
            sp.out_token[b] = d;
            if (sp.out_accepted) sp.out_accepted[b] = 1;
        }
        return;
    }

    // ---- rejected: race the residual
    uint64_t best = 0;
    float sstar = 0.0f;
    const uint32_t ng = (V + 3) >> 2;
    for (uint32_t g0 = 0; g0 < ng; g0 += kSpecThreads * kSpecUnroll) {
        float pv[kSpecUnroll][4], qv[kSpecUnroll][4];
#pragma unroll
        for (int k = 0; k < kSpecUnroll; ++k) {
            const uint32_t g = g0 + (uint32_t)k * kSpecThreads + t;
            if (sp.vec && g < ng) {
                const f32x4 a = __builtin_nontemporal_load((const f32x4*)P + g);
                const f32x4 c = __builtin_nontemporal_load((const f32x4*)Q + g);
                pv[k][0] = a.x; pv[k][1] = a.y; pv[k][2] = a.z; pv[k][3] = a.w;
                qv[k][0] = c.x; qv[k][1] = c.y; qv[k][2] = c.z; qv[k][3] = c.w;
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
#pragma unroll
        for (int k = 0; k < kSpecUnroll; ++k) {
            const uint32_t g = g0 + (uint32_t)k * kSpecThreads + t;
            float r[4];
            bool any = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                r[j] = pv[k][j] - qv[k][j];
                any |= r[j] > 0.0f;
            }
            if (!any) continue;
            const uint4 w4 = philox4x32_10(make_uint4(g, crow, sp.step_lo, sp.step_hi), klo, khi);
            const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
            // r / sstar * margin; with no score yet every candidate passes.
            const float kk = sstar > 0.0f ? __builtin_amdgcn_rcpf(sstar) * (1.0001f / (1.0f - 1e-4f)) : INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!(r[j] > 0.0f)) continue;
                const float w = fmaf((float)(0xFFFFFFFFu - words[j]), 0x1p-32f, 0x1p-33f);  // 1 - u <= E
                if (w > r[j] * kk) continue;
                const float s = r[j] / exp1_from_word(words[j]);
                const uint64_t pk = race_pack(s, 4 * g + (uint32_t)j);
                best = pk > best ? pk : best;
                sstar = fmaxf(sstar, s);
            }
        }
    }
    best = block_reduce<kSpecThreads>(best, MaxU64(), red);
    if (t == 0) {
        sp.out_token[b] = best ? (int32_t)~(uint32_t)best : -1;  // -1: nothing to resample (p is all zero)
        if (sp.out_accepted) sp.out_accepted[b] = 0;
    }
}

}  // namespace nucleus
