// rr_launch_util.hpp -- typed kernel launch that reports its own status.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <tuple>
#include <utility>

#include "../../include/rr.h"

namespace rr {

// Launch `k` with arguments converted to the kernel's parameter types and
// return RR_ERR_HIP if the runtime rejects the launch.  Using
// hipLaunchKernel's return code keeps errors from unrelated earlier calls
// out of this launch's status.
template <class... KArgs, class... Args>
rr_status launch_kernel(void (*k)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                        hipStream_t stream, Args&&... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> held(static_cast<KArgs>(std::forward<Args>(args))...);
    return std::apply(
        [&](auto&... a) {
            void* ptrs[] = {static_cast<void*>(&a)...};
            hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs,
                                           lds_bytes, stream);
            return e == hipSuccess ? RR_OK : RR_ERR_HIP;
        },
        held);
}

// Workgroups of kernel k resident per CU at nt threads and `lds` bytes of
// dynamic LDS.  The runtime's answer depends only on the kernel's resources,
// and asking costs microseconds of host time in front of every launch, so
// each (kernel, nt, lds) is asked once per process; the table holds a few
// dozen of them.
template <class K>
rr_status blocks_per_cu(K k, int nt, int* out, size_t lds = 0)
{
    struct Entry {
        const void* fn;
        int nt;
        size_t lds;
        int blocks;
    };
    static std::mutex mu;
    static Entry table[64];
    static int used = 0;
    const void* fn = reinterpret_cast<const void*>(k);
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (table[i].fn == fn && table[i].nt == nt && table[i].lds == lds) {
                *out = table[i].blocks;
                return RR_OK;
            }
    }
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k, nt, lds) != hipSuccess || v < 1)
        return RR_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (used < 64) table[used++] = Entry{fn, nt, lds, v};
    *out = v;
    return RR_OK;
}

}  // namespace rr
