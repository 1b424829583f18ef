// stream_read.h -- a read-only streaming kernel: every 16-byte unit of a
// buffer is loaded once (coalesced dwordx4, non-temporal) and folded into an
// XOR checksum.  It measures the HBM read ceiling on the same device, with the
// same load width the sampler uses, so the sampler's achieved bandwidth can
// be read against both the published peak and what a pure stream reaches.
#pragma once

#include "common.h"

namespace nucleus {

constexpr int kStreamBlock = 256;
constexpr int kStreamDepth = 16;  // 16-byte loads in flight per thread
constexpr int kStreamSinkSlots = 256;

// Block b reads the contiguous 64 KiB [b, b + 1) * 256 * 16 units of 16
// bytes, sixteen non-temporal dwordx4 loads per thread issued before any is
// used, each load instruction covering 4 KiB of consecutive addresses.  Of
// the grid-stride loops (1024..32768 blocks, 4..16 loads in flight,
// non-temporal or default policy) and contiguous-chunk blocks of 8 or 16
// loads per thread measured on MI355X over a 131 MB buffer, this shape read
// fastest; every launch has about 2000 blocks per 131 MB, eight per CU.
__global__ __launch_bounds__(kStreamBlock) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                                   const uint8_t* __restrict__ tail, int ntail,
                                                                   unsigned long long* sink)
{
    const size_t base = (size_t)blockIdx.x * (kStreamBlock * kStreamDepth) + threadIdx.x;
    uint32_t acc = 0;
    if (base + (size_t)(kStreamDepth - 1) * kStreamBlock < n16) {
        u32x4 v[kStreamDepth];
#pragma unroll
        for (int u = 0; u < kStreamDepth; ++u) v[u] = __builtin_nontemporal_load(buf + base + u * kStreamBlock);
#pragma unroll
        for (int u = 0; u < kStreamDepth; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    } else {
        for (int u = 0; u < kStreamDepth; ++u) {
            const size_t i = base + (size_t)u * kStreamBlock;
            if (i < n16) {
                const u32x4 v = __builtin_nontemporal_load(buf + i);
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            }
        }
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
    const size_t per_block = (size_t)kStreamBlock * kStreamDepth;
    size_t blocks = (n16 + per_block - 1) / per_block;
    if (blocks < 1) blocks = 1;
    if (blocks > 0x7FFFFFFFu) return false;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamBlock), 0, s, (const u32x4*)buf, n16,
                       (const uint8_t*)buf + n16 * 16, ntail, (unsigned long long*)sink);
    return hipGetLastError() == hipSuccess;
}

}  // namespace nucleus
