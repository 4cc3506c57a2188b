// Read-only streaming probe: the rate at which this chip moves a buffer of a
// given size from HBM to the CUs in one launch, with no compute and no
// writes beyond one word per work-group.  It measures the ceiling that the
// block attention's own streaming is compared with (a launch that reads one
// layer's cache, and a long one), so that "fraction of peak" can be read next
// to "fraction of what one launch of that size can reach".
#include "common.hpp"
#include "kernels.hpp"

#include "../../include/orthrus.h"

namespace orthrus {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;       // 16-byte loads in flight per lane

// Work-group w reads bytes [w*per, min((w+1)*per, n)) of src with 16-byte
// loads, kProbeUnroll in flight per lane, and folds them into one word.
__global__ void __launch_bounds__(kProbeThreads) stream_read_kernel(const u32x4* __restrict__ src,
                                                                  int64_t n16, int64_t per16,
                                                                  uint32_t* __restrict__ sink)
{
    const int64_t lo = (int64_t)blockIdx.x * per16;
    const int64_t hi = lo + per16 < n16 ? lo + per16 : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    constexpr int64_t STEP = (int64_t)kProbeThreads * kProbeUnroll;
    int64_t i = lo + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < hi; i += STEP) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * kProbeThreads];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < hi; i += kProbeThreads) acc ^= src[i];
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
    __shared__ uint32_t part[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" int orthrus_stream_read(const void *src, size_t bytes, int work_groups,
                                   uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink) return ORTHRUS_ERR_NULL;
    if (bytes < 16 || (bytes & 15u) || work_groups < 1) return ORTHRUS_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || work_groups > 65535)
        return ORTHRUS_ERR_UNSUPPORTED;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t per16 = (n16 + work_groups - 1) / work_groups;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)work_groups), dim3(kProbeThreads), 0,
                       stream, static_cast<const u32x4 *>(src), n16, per16, sink);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}
