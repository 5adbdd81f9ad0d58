// copy_probe.hip -- plain device copy used as the achievable-bandwidth
// reference for the memory-bound kernels and to calibrate the profiler's
// HBM byte counters (a copy of B bytes reads B and writes B).

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

constexpr int kUnroll = 1;

__global__ __launch_bounds__(kBlock) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                      int64_t n16, int64_t nblocks)
{
    const int64_t base = xcd_block(blockIdx.x, nblocks) * (kBlock * kUnroll) + threadIdx.x;
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n16)
            v[u] = ld_stream16(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kBlock;
        if (i < n16)
            st_stream16(dst + i, v[u]);
    }
}

}  // namespace

hipError_t launch_copy_probe(void* dst, const void* src, size_t bytes, hipStream_t stream)
{
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    const int64_t per_block = kBlock * kUnroll;
    int64_t nblocks = (n16 + per_block - 1) / per_block;
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    void* args[] = {&s, &d, const_cast<int64_t*>(&n16), &nblocks};
    return hipLaunchKernel(reinterpret_cast<const void*>(copy_kernel), dim3(static_cast<uint32_t>(nblocks)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace dq
