// rr_launch_util.hpp -- typed kernel launch that reports its own status.
#pragma once

#include <hip/hip_runtime.h>

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

}  // namespace rr
