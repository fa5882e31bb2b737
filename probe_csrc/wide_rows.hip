// Register-row RMSNorm geometries at N = 32768 for the measurement tools (not
// part of the library): the library's rownorm_regs_kernel layout (each lane
// holds its chunks of the row in VGPRs, 16-byte non-temporal loads and stores,
// one cross-wave LDS step) with the lanes per row, the occupancy cap, the XCD
// row runs and the point where the weight is loaded (with the row, or after
// the reduction) chosen per variant. Each launch records the kernel's own start
// and end in two events (hipExtLaunchKernel), as the library's timed entry
// points do.
#include <hip/hip_ext.h>

#include "../memory_bound_normalization_amd/csrc/rownorm.hip"

namespace mbn {
namespace {

template <int WPR, int MAXC, bool LATE_W>
__global__ void __launch_bounds__(64 * WPR) wide_regs_kernel(RowNormArgs a) {
  constexpr int TPR = 64 * WPR;
  __shared__ float part[2][WPR];
  const int nchunk = a.nchunk;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = xcd_remap(blockIdx.x, gridDim.x, a.xcd_group);
  if (row >= a.M) return;  // the grid has exactly M workgroups
  const int64_t base = row * nchunk;
  u32x4 xv[MAXC], wreg[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j)
    xv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x) + base + j * TPR + t);
  if constexpr (!LATE_W) {
#pragma unroll
    for (int j = 0; j < MAXC; ++j) wreg[j] = reinterpret_cast<const u32x4*>(a.w)[j * TPR + t];
  }
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = Bf16::lo(xv[j][e]);
      const float q = Bf16::hi(xv[j][e]);
      acc0 = __builtin_fmaf(p, p, acc0);
      acc1 = __builtin_fmaf(q, q, acc1);
    }
  }
  float s1[1] = {acc0 + acc1};
  rows_sum<WPR, 1>(s1, nullptr, &part[0][0], nchunk, t, wave, 0);
  const float scale = __builtin_amdgcn_rsqf(__builtin_fmaf(s1[0], a.inv_n, a.eps));
  if constexpr (LATE_W) {
#pragma unroll
    for (int j = 0; j < MAXC; ++j) wreg[j] = reinterpret_cast<const u32x4*>(a.w)[j * TPR + t];
  }
  u32x4* yrow = reinterpret_cast<u32x4*>(a.y) + base;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = Bf16::pack((Bf16::lo(xv[j][e]) * scale) * Bf16::lo(wreg[j][e]),
                        (Bf16::hi(xv[j][e]) * scale) * Bf16::hi(wreg[j][e]));
    store_nt_16(yrow + j * TPR + t, o);
  }
}

template <int WPR, int MAXC, bool LATE_W>
int wide_launch(const void* x, const void* w, void* y, int64_t M, float eps, int cap, int group, hipStream_t s,
                hipEvent_t e0, hipEvent_t e1) {
  constexpr int N = 32768;
  static_assert(64 * WPR * MAXC * 8 == N, "the lanes cover the row");
  RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = N / 8;
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  a.xcd_group = group;
  hipExtLaunchKernelGGL((wide_regs_kernel<WPR, MAXC, LATE_W>), dim3((unsigned)M), dim3(64 * WPR),
                        (std::uint32_t)rownorm_regs_lds_bytes(cap), s, e0, e1, 0u, a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace
}  // namespace mbn

extern "C" {

// Variant v of the sweep (see probe.py WIDE_ROW_VARIANTS) on x[M, 32768] bf16:
// 0 = ok, 1 = invalid arguments, 3 = launch failed.
__attribute__((visibility("default"))) int mbn_wide_rows_variant(const void* x, const void* w, void* y, int64_t M,
                                                                 float eps, int v, void* stream, void* e0, void* e1) {
  using namespace mbn;
  if (!x || !w || !y || M <= 0 || M > 0x7fffffffLL || !e0 || !e1) return 1;
  const hipStream_t s = (hipStream_t)stream;
  const hipEvent_t a = (hipEvent_t)e0, b = (hipEvent_t)e1;
  switch (v) {
    case 1: return wide_launch<16, 4, false>(x, w, y, M, eps, 4, 4, s, a, b);  // the table's entry
    case 2: return wide_launch<16, 4, true>(x, w, y, M, eps, 4, 4, s, a, b);
    case 3: return wide_launch<16, 4, true>(x, w, y, M, eps, 4, 0, s, a, b);
    case 4: return wide_launch<16, 4, true>(x, w, y, M, eps, 4, 8, s, a, b);
    case 5: return wide_launch<8, 8, false>(x, w, y, M, eps, 4, 4, s, a, b);
    case 6: return wide_launch<8, 8, false>(x, w, y, M, eps, 2, 4, s, a, b);
    case 7: return wide_launch<8, 8, true>(x, w, y, M, eps, 4, 4, s, a, b);
    case 8: return wide_launch<8, 8, true>(x, w, y, M, eps, 3, 4, s, a, b);
    case 9: return wide_launch<8, 8, true>(x, w, y, M, eps, 0, 4, s, a, b);
    case 10: return wide_launch<8, 8, true>(x, w, y, M, eps, 4, 0, s, a, b);
    case 11: return wide_launch<4, 16, true>(x, w, y, M, eps, 4, 4, s, a, b);
    case 12: return wide_launch<4, 16, true>(x, w, y, M, eps, 8, 4, s, a, b);
    default: return 1;
  }
}

}  // extern "C"
