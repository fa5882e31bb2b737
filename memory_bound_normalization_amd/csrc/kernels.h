// Host-side launchers of the gfx950 kernels. Arguments are already validated
// by the C entry points; each launcher enqueues one kernel on `stream` and
// returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbn {

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps,
                          hipStream_t stream);

hipError_t launch_qk_norm_rope(void* qkv, const void* q_w, const void* k_w,
                               const int64_t* positions, int64_t T, int n_q_heads,
                               int n_kv_heads, float eps, float theta, hipStream_t stream);

}  // namespace mbn
