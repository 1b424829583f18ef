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
};

}  // namespace nucleus
