// rr_stream.hip -- reference streams of known size: the achievable HBM
// bandwidth that the row kernels are compared with, beside the published peak.
//
// Plain 128-bit non-temporal passes with no arithmetic on the data: each
// workgroup takes one contiguous run of tiles (8 chunks of 16 bytes per
// thread per tile), so every workgroup streams one long sequential range;
// chunks past the last whole tile are taken grid-stride.
#include <hip/hip_runtime.h>

#include "../../include/rr.h"
#include "../../include/rr_test.h"
#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch_util.hpp"

namespace rr {

constexpr int kStreamUnroll = 8;

template <int MODE>
__global__ __launch_bounds__(kBlockThreads) void k_stream(const uint4* __restrict__ x,
                                                          uint4* __restrict__ y, int64_t n16)
{
    constexpr int64_t kTile = (int64_t)kStreamUnroll * kBlockThreads;
    const int64_t ntiles = n16 / kTile;
    const int64_t t_end = ((int64_t)blockIdx.x + 1) * ntiles / gridDim.x;
    uint32_t acc = 0;
    const uint4 pattern = make_uint4(blockIdx.x, threadIdx.x, 0x5eedu, 0u);
    for (int64_t t = (int64_t)blockIdx.x * ntiles / gridDim.x; t < t_end; ++t) {
        const int64_t base = t * kTile + threadIdx.x;
        uint4 v[kStreamUnroll];
        if constexpr (MODE != RR_TEST_STREAM_WRITE) {
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u)
                v[u] = load16_nt(x + base + (int64_t)u * kBlockThreads);
        }
        if constexpr (MODE == RR_TEST_STREAM_READ) {
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u)
                acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        } else {
#pragma unroll
            for (int u = 0; u < kStreamUnroll; ++u)
                store16_nt(y + base + (int64_t)u * kBlockThreads,
                           MODE == RR_TEST_STREAM_COPY ? v[u] : pattern);
        }
    }
    for (int64_t i = ntiles * kTile + (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kBlockThreads) {
        if constexpr (MODE == RR_TEST_STREAM_READ) {
            const uint4 u = load16_nt(x + i);
            acc ^= u.x ^ u.y ^ u.z ^ u.w;
        } else if constexpr (MODE == RR_TEST_STREAM_COPY) {
            store16_nt(y + i, load16_nt(x + i));
        } else {
            store16_nt(y + i, pattern);
        }
    }
    if constexpr (MODE == RR_TEST_STREAM_READ)
        asm volatile("" ::"v"(acc));  // the loads feed a value the compiler must keep
}

}  // namespace rr

extern "C" rr_status rr_test_stream(int32_t mode, const void* x, void* y, size_t bytes,
                                    int32_t blocks_per_cu, void* stream)
{
    using namespace rr;
    if (mode != RR_TEST_STREAM_READ && mode != RR_TEST_STREAM_WRITE && mode != RR_TEST_STREAM_COPY)
        return RR_ERR_SHAPE;
    if ((mode != RR_TEST_STREAM_WRITE && !x) || (mode != RR_TEST_STREAM_READ && !y))
        return RR_ERR_NULL;
    if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(x) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(y) % 16 != 0)
        return RR_ERR_SHAPE;
    if (blocks_per_cu == 0)
        blocks_per_cu = 2;
    if (blocks_per_cu < 1 || blocks_per_cu > 16)
        return RR_ERR_SHAPE;
    if (bytes == 0)
        return RR_OK;
    int32_t cu = 0;
    const rr_status st = rr_device_cu_count(&cu);
    if (st != RR_OK)
        return st;
    const dim3 grid((unsigned)(blocks_per_cu * cu)), block(kBlockThreads);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n16 = (int64_t)(bytes / 16);
    const uint4* xs = static_cast<const uint4*>(x);
    uint4* ys = static_cast<uint4*>(y);
    switch (mode) {
    case RR_TEST_STREAM_READ: return launch_kernel(k_stream<RR_TEST_STREAM_READ>, grid, block, 0, s, xs, ys, n16);
    case RR_TEST_STREAM_WRITE: return launch_kernel(k_stream<RR_TEST_STREAM_WRITE>, grid, block, 0, s, xs, ys, n16);
    default: return launch_kernel(k_stream<RR_TEST_STREAM_COPY>, grid, block, 0, s, xs, ys, n16);
    }
}
