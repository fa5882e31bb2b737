// Register-row geometries for small row-norm launches, for the measurement
// tools (not part of the library): the library's rownorm_regs_kernel (RMSNorm,
// residual add + RMSNorm, LayerNorm or L2Norm) at widths 2048 ... 16384 with
// the lanes per row, rows per workgroup and chunks per lane chosen per
// variant, launched plainly or, given two events, with the kernel's own start
// and end recorded in them (hipExtLaunchKernel).
#include <hip/hip_ext.h>

#include "../memory_bound_normalization_amd/csrc/rownorm.hip"

namespace mbn {
namespace {

template <Norm MODE, int WPR, int ROWS, int MAXC>
int small_launch(const RowNormArgs& args, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int64_t N = (int64_t)args.nchunk * 8;
  if (N != (int64_t)64 * WPR * MAXC * 8) return 1;
  RowNormArgs a = args;
  a.inv_n = 1.0f / (float)N;
  a.xcd_group = 0;
  const int64_t blocks = (a.M + ROWS - 1) / ROWS;
  if (e0)
    hipExtLaunchKernelGGL((rownorm_regs_kernel<MODE, Bf16, WPR, ROWS, MAXC, true>), dim3((unsigned)blocks),
                          dim3(64 * WPR * ROWS), 0u, s, e0, e1, 0u, a);
  else
    hipLaunchKernelGGL((rownorm_regs_kernel<MODE, Bf16, WPR, ROWS, MAXC, true>), dim3((unsigned)blocks),
                       dim3(64 * WPR * ROWS), 0u, s, a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

typedef int (*SmallLaunch)(const RowNormArgs&, hipStream_t, hipEvent_t, hipEvent_t);
struct SmallVariant {
  int wpr, rows, maxc;
  SmallLaunch f[4];  // by mode: RMSNorm, residual add + RMSNorm, LayerNorm, L2Norm
};
#define MBN_SMALL(W, R, C)                                                                             \
  SmallVariant {                                                                                       \
    W, R, C, {&small_launch<Norm::kRms, W, R, C>, &small_launch<Norm::kAddRms, W, R, C>,               \
              &small_launch<Norm::kLayer, W, R, C>, &small_launch<Norm::kL2, W, R, C>}                 \
  }
// Index order is the variant number; the width is 64 * wpr * maxc * 8.
const SmallVariant kSmall[] = {
    MBN_SMALL(1, 1, 4), MBN_SMALL(1, 2, 4), MBN_SMALL(1, 4, 4), MBN_SMALL(2, 1, 2), MBN_SMALL(2, 2, 2),
    MBN_SMALL(4, 1, 1),                                                                              // 2048
    MBN_SMALL(1, 1, 8), MBN_SMALL(1, 2, 8), MBN_SMALL(2, 1, 4), MBN_SMALL(2, 2, 4), MBN_SMALL(4, 1, 2),
    MBN_SMALL(4, 2, 2), MBN_SMALL(8, 1, 1),                                                          // 4096
    MBN_SMALL(2, 1, 8), MBN_SMALL(2, 2, 8), MBN_SMALL(4, 1, 4), MBN_SMALL(4, 2, 4), MBN_SMALL(8, 1, 2),
    MBN_SMALL(16, 1, 1),                                                                             // 8192
    MBN_SMALL(4, 1, 8), MBN_SMALL(8, 1, 4), MBN_SMALL(16, 1, 2), MBN_SMALL(4, 2, 8), MBN_SMALL(8, 2, 4),  // 16384
};

}  // namespace
}  // namespace mbn

extern "C" {

__attribute__((visibility("default"))) int mbn_small_regs_count() {
  return (int)(sizeof(mbn::kSmall) / sizeof(mbn::kSmall[0]));
}

// Geometry of variant v: {lanes per row / 64, rows per workgroup, chunks per lane}.
__attribute__((visibility("default"))) int mbn_small_regs_geometry(int v, int* out) {
  if (v < 0 || v >= mbn_small_regs_count() || !out) return 1;
  out[0] = mbn::kSmall[v].wpr;
  out[1] = mbn::kSmall[v].rows;
  out[2] = mbn::kSmall[v].maxc;
  return 0;
}

// Row norm `mode` (0 RMSNorm, 1 residual add + RMSNorm, 2 LayerNorm, 3 L2Norm)
// of bf16 rows [M, N] with variant v (N must be its width); r and h only for
// mode 1, w for all but mode 3, b for mode 2 (else null); e0 and e1 both
// events or both null. 0 = ok, 1 = invalid arguments, 3 = launch failed.
__attribute__((visibility("default"))) int mbn_small_regs(int mode, const void* x, const void* r, const void* w,
                                                          const void* b, void* h, void* y, int64_t M, int64_t N,
                                                          float eps, int v, void* stream, void* e0, void* e1) {
  if (mode < 0 || mode > 3 || !x || !y || M <= 0 || M > (1 << 20) || N <= 0 || N % 8 != 0 || v < 0 ||
      v >= mbn_small_regs_count() || !e0 != !e1)
    return 1;
  if ((mode != 3 && !w) || (mode == 2 && !b) || (mode == 1 && (!r || !h))) return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.r = static_cast<const uint16_t*>(r);
  a.w = static_cast<const uint16_t*>(w);
  a.b = static_cast<const uint16_t*>(b);
  a.h = static_cast<uint16_t*>(h);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.eps = eps;
  return mbn::kSmall[v].f[mode](a, (hipStream_t)stream, (hipEvent_t)e0, (hipEvent_t)e1);
}

}  // extern "C"
