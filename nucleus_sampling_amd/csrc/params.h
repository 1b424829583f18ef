// params.h -- launch parameters passed by value to the sampler's kernels.
#pragma once

#include <stdint.h>

namespace nucleus {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

struct Params {
    const void* logits;       // [B, stride] elements of the launch dtype
    int64_t B, V, stride;
    const float* temperature; // [B]
    const float* top_p;       // [B]
    const int32_t* top_k;     // [B] or null
    const float* min_p;       // [B] or null
    uint32_t seed_lo, seed_hi, step_lo, step_hi;
    int32_t* out_token;       // [B]
    int32_t* out_count;       // [B]
    float* out_probs;         // [B, V] or null
    float* out_min_kept;      // [B] or null
    int vec_in;               // rows start 16-byte (f32) / 8-byte (bf16) aligned
    const uint64_t* seeds;    // [B] per-row race keys, or null (every row uses seed_lo/hi)
    float* out_logprobs;      // [B, V] or null
    // The pre-chain (penalties, grammar mask); read only by row_kernel<..., true>.
    const int32_t* hist;      // [B, hist_len] token ids, -1 padded, or null
    int64_t hist_len;
    const float* rep_pen;     // [B] or null (1)
    const float* freq_pen;    // [B] or null (0)
    const float* pres_pen;    // [B] or null (0)
    const uint32_t* allowed;  // [B, ceil(V/32)] bit masks, or null (all allowed)
    uint64_t* stamps;         // [B, kStamps] phase clocks (builds with NUCLEUS_PHASE_STAMPS), or null
};

// Phase clocks of the one-workgroup-per-row kernel, compiled in only with
// NUCLEUS_PHASE_STAMPS: thread 0 of row b's workgroup writes the 100 MHz
// constant-rate clock at each phase boundary to stamps[b * kStamps + k]
// (k < 8), and a few facts about the row after them.
constexpr int kStamps = 16;
enum StampPoint {
    kStampStart = 0,     // the workgroup starts
    kStampPass1 = 1,     // pass 1 (max, error flag, fused histogram) done
    kStampHist = 2,      // the row's bins are ready (window folded, or pass 2 done)
    kStampDecide = 3,    // decide done
    kStampClassify = 4,  // classify done
    kStampPass3 = 5,     // pass 3 (race of the surely kept tokens, candidates) done
    kStampResolve = 6,   // resolver done, outputs written
    kStampProbs = 7,     // probability pass done (or skipped)
    kStampMode = 8,      // (facts) the row's mode after decide
    kStampCands = 9,     // crossing-bin candidates listed after pass 3
    kStampMarked = 10,   // marked runs of groups holding them
};

#ifdef NUCLEUS_PHASE_STAMPS
__device__ __forceinline__ void phase_stamp(const Params& p, int64_t b, int k)
{
    if (p.stamps && threadIdx.x == 0) p.stamps[b * kStamps + k] = wall_clock64();
}
__device__ __forceinline__ void phase_fact(const Params& p, int64_t b, int k, uint64_t v)
{
    if (p.stamps && threadIdx.x == 0) p.stamps[b * kStamps + k] = v;
}
#else
__device__ __forceinline__ void phase_stamp(const Params&, int64_t, int) {}
__device__ __forceinline__ void phase_fact(const Params&, int64_t, int, uint64_t) {}
#endif

}  // namespace nucleus
