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
};

}  // namespace nucleus
