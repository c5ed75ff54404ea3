// Shared by the library's translation units; not part of the C ABI.
#ifndef FA_INTERNAL_H
#define FA_INTERNAL_H

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

#include "fa.h"

namespace fa_detail {
// HIP error code behind the calling thread's last FA_ERR_HIP.
extern thread_local int g_last_hip;

// FA_OK, or FA_ERR_HIP after recording `err` for fa_last_hip_error().
inline int status_of(hipError_t err) {
    if (err == hipSuccess) return FA_OK;
    g_last_hip = (int)err;
    return FA_ERR_HIP;
}

template <class... KArgs, size_t... I>
int launch_tuple(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, std::tuple<KArgs...>& vals,
                 std::index_sequence<I...>) {
    void* argv[] = {static_cast<void*>(&std::get<I>(vals))...};
    return status_of(hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream));
}

// Enqueue kernel<<<grid, block, 0, stream>>>(args...) and return the status of
// this launch alone.  hipLaunchKernel reports the error of the launch it
// makes; the thread's pending error state (for instance hipErrorNotReady left
// by an earlier hipStreamQuery) is neither read nor cleared.
template <class... KArgs, class... Args>
int launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> vals(args...);
    return launch_tuple(kernel, grid, block, stream, vals, std::index_sequence_for<KArgs...>{});
}
}  // namespace fa_detail

#endif
