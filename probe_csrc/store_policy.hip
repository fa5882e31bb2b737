// The library's one-shot row-norm kernel with another cache policy on its
// output stores, for the measurement tools (not part of the library). probe.py
// writes gen/rownorm_store_policy.hip: the library's csrc/rownorm.hip with the
// one-shot kernel's output store (pass 2 of rownorm_block) replaced by
// MBN_STORE_Y, defined here as a global_store_dwordx4 carrying the nt / sc0 /
// sc1 bits of MBN_PROBE_POLICY (0: nt, the library's own policy but through
// inline assembly; 1: nt sc1; 2: sc1; 3: sc0 sc1). Nothing else changes.
//
// The stores are inline assembly, each followed by two wait states (on gfx950
// a VALU instruction may overwrite the data registers of a store wider than 8
// bytes only two wait states after it; the compiler inserts them after its own
// stores, not after inline assembly). They are pass 2's stores: by then every
// load of the workgroup has completed (pass 1 waited for all of them), so the
// compiler's vector-memory waits, which do not count these stores, have
// nothing left to wait for.
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef MBN_PROBE_POLICY
#define MBN_PROBE_POLICY 1
#endif
#if MBN_PROBE_POLICY == 0
#define MBN_PROBE_POLICY_BITS "nt"
#elif MBN_PROBE_POLICY == 1
#define MBN_PROBE_POLICY_BITS "nt sc1"
#elif MBN_PROBE_POLICY == 2
#define MBN_PROBE_POLICY_BITS "sc1"
#elif MBN_PROBE_POLICY == 3
#define MBN_PROBE_POLICY_BITS "sc0 sc1"
#else
#error "MBN_PROBE_POLICY is 0-3"
#endif

#define MBN_STORE_Y(p, v)                                                                                   \
  __asm__ __volatile__("global_store_dwordx4 %0, %1, off " MBN_PROBE_POLICY_BITS "\n\ts_nop 1" ::"v"(p), \
                       "v"(v))

#include "rownorm_store_policy.hip"

extern "C" {

// RMSNorm, bf16, N = 16384, at the library's table entry for that width (two
// waves per row, two rows per workgroup, per-chunk waits, occupancy cap 2,
// XCD row groups of 4). 0 = ok, 1 = other shape or grid too large, 3 = launch
// failed.
__attribute__((visibility("default"))) int mbn_sp_rmsnorm(const void* x, const void* w, void* y, int64_t M,
                                                          int64_t N, float eps, void* stream) {
  constexpr int WPR = 2, ROWS = 2, RPL = 1, MAXC = 16;
  if (N != 16384 || M <= 0 || !x || !w || !y) return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  a.xcd_group = 4;
  const int64_t blocks = (M + ROWS * RPL - 1) / (ROWS * RPL);
  if (blocks * 64 * WPR * ROWS > 0xffffffffLL) return 1;
  const size_t lds = mbn::rownorm_lds_bytes(ROWS * RPL, N, 2);
  hipLaunchKernelGGL((mbn::rownorm_kernel<mbn::Norm::kRms, mbn::Bf16, WPR, ROWS, RPL, MAXC, true, true>),
                     dim3((unsigned)blocks), dim3(64 * WPR * ROWS), lds, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
