// Host-side launchers of the gfx950 kernels. Arguments are already validated
// by the C entry points; each launcher enqueues its kernel on `stream` (as
// several launches over consecutive rows or tokens when one dispatch would
// exceed kMaxWorkItems) and returns the launch status.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbn {

// Kernel-execution timestamps for one entry-point call. While a call of a
// *_timed entry point runs, the calling thread's slot points at its events:
// the call's first dispatch records `start` when its kernel starts and every
// dispatch records `stop` when its kernel ends (hipExtLaunchKernel), so that
// stop - start spans exactly the call's kernels, without the queue packets a
// hipEventRecord before and after the call would add to the interval. Null
// (every other call): plain launches.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
};
inline LaunchTiming*& launch_timing() {
  static thread_local LaunchTiming* slot = nullptr;
  return slot;
}

// Every kernel launch of the library goes through here; returns the launch status.
template <typename... KArgs, typename... Args>
hipError_t dispatch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                    Args... args) {
  LaunchTiming* t = launch_timing();
  if (!t) {
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, static_cast<KArgs>(args)...);
  } else {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, stream, t->start, t->stop, 0u,
                          static_cast<KArgs>(args)...);
    t->start = nullptr;  // later dispatches of the same call only move `stop`
  }
  return hipGetLastError();
}

// Work-items of one dispatch: the grid size fields of an HSA kernel dispatch
// packet are 32-bit, so a one-dimensional launch covers at most 2^32 - 1.
constexpr int64_t kMaxWorkItems = 0xffffffffLL;

// Storage type of every 16-bit tensor of a call.
enum class Storage : int { kBf16 = 0, kF16 = 1 };

// Row-wise norms served by one kernel template (rownorm.hip).
enum class Norm : int { kRms = 0, kAddRms = 1, kLayer = 2, kL2 = 3 };

// Kernel arguments of every row norm; unused pointers are null.
struct RowNormArgs {
  const uint16_t* x;  // [M, N] input (16-bit storage type of the call)
  const uint16_t* r;  // [M, N] residual (kAddRms)
  const uint16_t* w;  // [N] weight (all but kL2)
  const uint16_t* b;  // [N] bias (kLayer)
  uint16_t* h;        // [M, N] x + r (kAddRms)
  uint16_t* y;        // [M, N] output
  int64_t M;
  int nchunk;         // N / 8
  float inv_n;        // 1 / N, set by the launcher
  float eps;
  int xcd_group;      // set by the launcher
};

// Which row-norm kernel serves a launch: kAuto picks by width and row count;
// the others force a path (tuning tools; kPersistent fails with
// hipErrorInvalidValue for widths or modes it does not serve). grid > 0
// overrides the persistent grid size.
enum class RowNormPath : int { kAuto = 0, kOneShot = 1, kPersistent = 2 };

hipError_t launch_rownorm(Norm mode, Storage dtype, RowNormArgs args, hipStream_t stream,
                          RowNormPath path = RowNormPath::kAuto, int grid = 0);

// Arguments of the any-width row norms (rownorm_any.hip): pointers need only
// 2-byte alignment and N may be any width up to MBN_RMSNORM_MAX_N.
struct RowNormAnyArgs {
  const uint16_t* x;
  const uint16_t* r;
  const uint16_t* w;
  const uint16_t* b;
  uint16_t* h;
  uint16_t* y;
  int64_t M;
  int n;          // N
  float inv_n;    // set by the launcher
  float eps;
  int xcd_group;  // set by the launcher (row blocks per XCD run, 16-byte staged kernels)
};

hipError_t launch_rownorm_any(Norm mode, Storage dtype, RowNormAnyArgs args, hipStream_t stream);

// Elements per access (4, 2 or 1) the any-width kernels use for these
// arguments: the widest group that divides N and every pointer's alignment.
int rownorm_any_group(const RowNormAnyArgs& args);

// Dynamic LDS bytes a row-norm launch requests (exposed for tuning tools).
size_t rownorm_lds_bytes(int rows, int64_t N, int wgs_per_cu);
size_t rownorm_regs_lds_bytes(int wgs_per_cu);

// rotary_dim: a multiple of 16 in [16, 128]; 128 is the full-rotary case.
hipError_t launch_qk_norm_rope(Storage dtype, void* qkv, const void* q_w, const void* k_w,
                               const int64_t* positions, int64_t T, int n_q_heads,
                               int n_kv_heads, int rotary_dim, float eps, float theta,
                               hipStream_t stream);

}  // namespace mbn
