// Launch-table entries the library used before, for the measurement tools
// (not part of the library): the library's own kernels from its source, at
// the entries that later measurements replaced, so that old and new can be
// timed side by side on the same data.
//
// mbn_lds_rmsnorm: the staged-row (LDS) kernel at N = 32768 and 65536, whose
// rows the tables now hold in VGPRs (1024 lanes per row, one row per
// workgroup, no occupancy cap, no XCD row groups, per-chunk waits on grids of
// at least 1024 workgroups).
//
// mbn_early_w_rmsnorm: the N <= 8192 band's previous entry (256 lanes per
// row, four chunks per lane, occupancy cap 4, XCD row groups of 8), which
// loads the weight alongside the row copy; the band now uses 512 lanes with
// the weight loaded after the reduction.
#include "../memory_bound_normalization_amd/csrc/rownorm.hip"

namespace {

template <int MAXC>
int launch_lds_rows(const void* x, const void* w, void* y, int64_t M, float eps, hipStream_t s) {
  constexpr int WPR = 16;
  constexpr int64_t N = (int64_t)64 * WPR * MAXC * 8;
  if (M <= 0 || M * 64 * WPR > 0xffffffffLL) return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  a.xcd_group = 0;
  const size_t lds = mbn::rownorm_lds_bytes(1, N, 0);
  if (M >= 1024)  // the launcher's threshold for the per-chunk-wait kernel
    hipLaunchKernelGGL((mbn::rownorm_kernel<mbn::Norm::kRms, mbn::Bf16, WPR, 1, 1, MAXC, true, true>),
                       dim3((unsigned)M), dim3(64 * WPR), lds, s, a);
  else
    hipLaunchKernelGGL((mbn::rownorm_kernel<mbn::Norm::kRms, mbn::Bf16, WPR, 1, 1, MAXC, true, false>),
                       dim3((unsigned)M), dim3(64 * WPR), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

template <bool FULL>
int launch_early_w(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps, hipStream_t s) {
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  a.xcd_group = 8;
  hipLaunchKernelGGL((mbn::rownorm_kernel<mbn::Norm::kRms, mbn::Bf16, 4, 1, 1, 4, FULL, false>), dim3((unsigned)M),
                     dim3(256), mbn::rownorm_lds_bytes(1, N, 4), s, a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace

extern "C" {

// RMSNorm, bf16, 4096 < N <= 8192 with N % 8 == 0 (the band's previous
// entry; it serves every width of the band). 0 = ok, 1 = other width or bad
// arguments, 3 = launch failed.
__attribute__((visibility("default"))) int mbn_early_w_rmsnorm(const void* x, const void* w, void* y, int64_t M,
                                                               int64_t N, float eps, void* stream) {
  if (!x || !w || !y || M <= 0 || M > 0x7fffffff || N <= 4096 || N > 8192 || N % 8) return 1;
  if (N == 8192) return launch_early_w<true>(x, w, y, M, N, eps, (hipStream_t)stream);
  return launch_early_w<false>(x, w, y, M, N, eps, (hipStream_t)stream);
}

// RMSNorm, bf16, N = 32768 or 65536 only. 0 = ok, 1 = other width or bad
// arguments, 3 = launch failed.
__attribute__((visibility("default"))) int mbn_lds_rmsnorm(const void* x, const void* w, void* y, int64_t M,
                                                           int64_t N, float eps, void* stream) {
  if (!x || !w || !y) return 1;
  if (N == 32768) return launch_lds_rows<4>(x, w, y, M, eps, (hipStream_t)stream);
  if (N == 65536) return launch_lds_rows<8>(x, w, y, M, eps, (hipStream_t)stream);
  return 1;
}

}  // extern "C"
