// Row-wise RMSNorm forward for gfx950, one row staged in LDS per row slot.
//
// The method ("[Inductor] Codegen Gluon", section 3.1): x is needed twice, for
// the x*x accumulation and for x * rstd * weight, so each row is read from HBM
// once into on-chip memory, kept narrow (bf16) there, and widened to fp32 only
// where it is computed on. On gfx950 the row copy is a burst of
// global_load_lds_dwordx4 (HBM -> LDS without passing through VGPRs), issued
// for the whole row before the first wait, so a workgroup keeps its entire row
// in flight.
//
// Work decomposition: a workgroup holds ROWS row slots; each row is served by
// WPR waves (64 * WPR lanes). Lane t of a row owns the 16-byte chunks
// k = j * (64 * WPR) + t, j < MAXC, and reads back only the chunks it loaded,
// so the two LDS passes need no barrier; the single barrier is the cross-wave
// step of the sum of squares. That step needs one float per wave of LDS; rather
// than allocate it beside the row (LDS is allocated in coarse granules, and
// 16 extra bytes on a 32 KiB row would cost one resident workgroup per CU), each
// lane keeps its first chunk in VGPRs after pass 1 and the wave parks its
// partial sum in that chunk's LDS slot, which nothing reads afterwards. The LDS
// footprint is exactly ROWS * N * 2 bytes.
#include "device.h"
#include "kernels.h"

namespace mbn {
namespace {

// FULL: the row is exactly MAXC chunks per lane (the power-of-two widths), so
// no chunk needs a bounds predicate.
template <int WPR, int ROWS, int MAXC, bool FULL>
__global__ void __launch_bounds__(64 * WPR * ROWS)
rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
               uint16_t* __restrict__ y, int64_t M, int nchunk, float inv_n, float eps) {
  constexpr int TPR = 64 * WPR;  // lanes per row
  extern __shared__ u32x4 lds_rows[];  // ROWS * nchunk chunks of 16 bytes

  const int tid = threadIdx.x;
  const int slot = tid / TPR;
  const int t = tid - slot * TPR;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t row = (int64_t)blockIdx.x * ROWS + slot;
  const bool live = row < M;

  u32x4* buf = lds_rows + (size_t)slot * nchunk;
  const u32x4* xrow = reinterpret_cast<const u32x4*>(x) + row * nchunk;
  const u32x4* w4 = reinterpret_cast<const u32x4*>(w);

  // HBM -> LDS: the whole row, all chunks in flight before any wait.
  if (live) {
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if (FULL || k < nchunk)
        load_lds_16(xrow + k, (lds_void*)(buf + j * TPR + wave * 64));
    }
  }
  // Weights go to registers (an L2 hit after the first rows), overlapping the row.
  u32x4 wreg[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * TPR + t;
    wreg[j] = (FULL || k < nchunk) ? w4[k] : u32x4{0u, 0u, 0u, 0u};
  }
  wait_vmem();

  // Pass 1 (from LDS): sum of squares in fp32.
  float acc0 = 0.f, acc1 = 0.f;
  u32x4 first = {0u, 0u, 0u, 0u};  // chunk j = 0, kept for pass 2
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * TPR + t;
    if (FULL || k < nchunk) {
      const u32x4 v = buf[k];
      if (j == 0) first = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_lo(v[e]);
        const float b = bf16_hi(v[e]);
        acc0 = __builtin_fmaf(a, a, acc0);
        acc1 = __builtin_fmaf(b, b, acc1);
      }
    }
  }
  float ss = wave_sum(acc0 + acc1);
  if constexpr (WPR > 1) {
    // Chunk wave * 64 (lane 0's first chunk) is in VGPRs now and is not read
    // from LDS again; the launch table guarantees nchunk >= 64 * WPR here, so
    // every wave owns such a chunk.
    float* parked = reinterpret_cast<float*>(buf);
    if ((t & 63) == 0) parked[wave * 256] = ss;  // 256 floats = 64 chunks
    __syncthreads();
    ss = 0.f;
#pragma unroll
    for (int i = 0; i < WPR; ++i) ss += parked[i * 256];
  }
  const float rstd = __builtin_amdgcn_rsqf(__builtin_fmaf(ss, inv_n, eps));

  // Pass 2 (from LDS): y = x * rstd * w, rounded to bf16, streaming stores.
  if (live) {
    u32x4* yrow = reinterpret_cast<u32x4*>(y) + row * nchunk;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * TPR + t;
      if (FULL || k < nchunk) {
        const u32x4 v = (j == 0) ? first : buf[k];
        const u32x4 wv = wreg[j];
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = (bf16_lo(v[e]) * rstd) * bf16_lo(wv[e]);
          const float b = (bf16_hi(v[e]) * rstd) * bf16_hi(wv[e]);
          o[e] = pack_bf16x2(a, b);
        }
        store_nt_16(yrow + k, o);
      }
    }
  }
}

typedef void (*RmsKernel)(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, float, float);

struct RmsCfg {
  int max_nchunk;  // widest row (in 16-byte chunks) this entry serves
  int wpr, rows, maxc;
  RmsKernel ragged;  // any width up to max_nchunk
  RmsKernel full;    // width exactly max_nchunk
};

#define MBN_RMS_CFG(WPR, ROWS, MAXC)                                               \
  RmsCfg {                                                                         \
    64 * (WPR) * (MAXC), WPR, ROWS, MAXC, &rmsnorm_kernel<WPR, ROWS, MAXC, false>, \
        &rmsnorm_kernel<WPR, ROWS, MAXC, true>                                     \
  }

// Per-width launch table, narrowest first: the first entry whose max_nchunk
// covers the row is used. Every entry with WPR > 1 starts where the previous
// entry ends, at or above 64 * WPR chunks, which the parked partial sums need.
const RmsCfg kRmsTable[] = {
    MBN_RMS_CFG(1, 4, 1),   // N <= 512
    MBN_RMS_CFG(1, 4, 2),   // N <= 1024
    MBN_RMS_CFG(1, 4, 4),   // N <= 2048
    MBN_RMS_CFG(4, 1, 2),   // N <= 4096
    MBN_RMS_CFG(4, 1, 4),   // N <= 8192
    MBN_RMS_CFG(4, 1, 8),   // N <= 16384
    MBN_RMS_CFG(8, 1, 8),   // N <= 32768
    MBN_RMS_CFG(16, 1, 8),  // N <= 65536
};

}  // namespace

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps,
                          hipStream_t stream) {
  const int nchunk = (int)(N / 8);
  const RmsCfg* cfg = nullptr;
  for (const RmsCfg& c : kRmsTable)
    if (nchunk <= c.max_nchunk) { cfg = &c; break; }
  if (!cfg) return hipErrorInvalidValue;
  if (cfg->wpr > 1 && nchunk < 64 * cfg->wpr) return hipErrorInvalidValue;  // table invariant
  const int64_t blocks = (M + cfg->rows - 1) / cfg->rows;
  const size_t lds = (size_t)cfg->rows * (size_t)N * 2;
  const float inv_n = 1.0f / (float)N;
  const RmsKernel kernel = (nchunk == cfg->max_nchunk) ? cfg->full : cfg->ragged;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * cfg->wpr * cfg->rows), lds,
                     stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                     static_cast<uint16_t*>(y), M, nchunk, inv_n, eps);
  return hipGetLastError();
}

}  // namespace mbn
