// Shared by the library's translation units; not part of the C ABI.
#ifndef FA_INTERNAL_H
#define FA_INTERNAL_H

namespace fa_detail {
// HIP error code behind the calling thread's last FA_ERR_HIP.
extern thread_local int g_last_hip;
// FA_OK, or FA_ERR_HIP after recording hipGetLastError() for fa_last_hip_error().
int launch_status();
}  // namespace fa_detail

#endif
