// stream_read.h -- a read-only streaming kernel: every 16-byte unit of a
// buffer is loaded once (coalesced dwordx4, non-temporal) and folded into a
// checksum.  It measures the HBM read ceiling on the same device, with the
// same load width the sampler uses, so the sampler's achieved bandwidth can
// be read against both the published peak and what a pure stream reaches.
#pragma once

#include "common.h"

namespace nucleus {

constexpr int kStreamBlock = 256;
constexpr int kStreamUnroll = 4;
constexpr int kStreamSinkSlots = 256;

__global__ __launch_bounds__(kStreamBlock) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                                   const uint8_t* __restrict__ tail, int ntail,
                                                                   unsigned long long* sink)
{
    const size_t stride = (size_t)gridDim.x * kStreamBlock;
    size_t i = (size_t)blockIdx.x * kStreamBlock + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) acc ^= tail[threadIdx.x];
    acc = wave_reduce(acc, [](uint32_t a, uint32_t b) { return a ^ b; });
    // Spread the fold over kStreamSinkSlots words so that blocks do not queue
    // on one address.
    if ((threadIdx.x & (kWave - 1)) == 0 && acc)
        atomicXor(sink + (blockIdx.x % kStreamSinkSlots), (unsigned long long)acc);
}

inline bool launch_stream_read(const void* buf, size_t bytes, uint64_t* sink, hipStream_t s)
{
    const size_t n16 = bytes / 16;
    const int ntail = (int)(bytes % 16);
    size_t blocks = (n16 + (size_t)kStreamBlock * kStreamUnroll - 1) / ((size_t)kStreamBlock * kStreamUnroll);
    if (blocks < 1) blocks = 1;
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamBlock), 0, s, (const u32x4*)buf, n16,
                       (const uint8_t*)buf + n16 * 16, ntail, (unsigned long long*)sink);
    return hipGetLastError() == hipSuccess;
}

}  // namespace nucleus
