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

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b mod 8). With xcd_group = G > 0, XCD x is given runs of G consecutive
// row blocks instead of every 8th one, which changes how the concurrent HBM
// traffic of the XCDs interleaves; G = 0 keeps the identity. The remap is a
// bijection on the leading blocks that fill whole groups of 8*G; the rest keep
// their own index.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nblocks, int group) {
  if (group <= 0) return b;
  const int64_t span = 8 * (int64_t)group;
  if (b >= (nblocks / span) * span) return b;
  const int64_t xcd = b & 7, i = b >> 3;
  return (i / group) * span + xcd * group + (i % group);
}

// FULL: the row is exactly MAXC chunks per lane (the power-of-two widths), so
// no chunk needs a bounds predicate.
template <int WPR, int ROWS, int MAXC, bool FULL>
__global__ void __launch_bounds__(64 * WPR * ROWS)
rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
               uint16_t* __restrict__ y, int64_t M, int nchunk, float inv_n, float eps,
               int xcd_group) {
  constexpr int TPR = 64 * WPR;  // lanes per row
  extern __shared__ u32x4 lds_rows[];  // ROWS * nchunk chunks of 16 bytes (or more, see launcher)

  const int tid = threadIdx.x;
  const int slot = tid / TPR;
  const int t = tid - slot * TPR;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t block = xcd_remap(blockIdx.x, gridDim.x, xcd_group);
  const int64_t row = block * ROWS + slot;
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

typedef void (*RmsKernel)(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, float, float,
                          int);

// LDS of one CU on gfx950; a workgroup may use all of it.
constexpr size_t kLdsPerCU = 160 * 1024;

struct RmsCfg {
  int max_nchunk;    // widest row (in 16-byte chunks) this entry serves
  int wpr, rows, maxc;
  int wgs_per_cu;    // occupancy cap (0 = as many as LDS and waves allow)
  int xcd_group;     // row blocks per XCD run (0 = dispatch order)
  RmsKernel ragged;  // any width up to max_nchunk
  RmsKernel full;    // width exactly max_nchunk
};

#define MBN_RMS_CFG(WPR, ROWS, MAXC, CAP, GROUP)                                        \
  RmsCfg {                                                                              \
    64 * (WPR) * (MAXC), WPR, ROWS, MAXC, CAP, GROUP,                                   \
        &rmsnorm_kernel<WPR, ROWS, MAXC, false>, &rmsnorm_kernel<WPR, ROWS, MAXC, true> \
  }

// Per-width launch table, narrowest first: the first entry whose max_nchunk
// covers the row is used. Every entry with WPR > 1 starts where the previous
// entry ends, at or above 64 * WPR chunks, which the parked partial sums need.
// Entries for N = 4096 ... 32768 were chosen by timing every shape / cap /
// group combination on MI355X at M*N = 2^26 ... 2^28 (median of 7 repeats);
// the narrower and wider bands are untuned.
const RmsCfg kRmsTable[] = {
    MBN_RMS_CFG(1, 4, 1, 0, 0),    // N <= 512
    MBN_RMS_CFG(1, 4, 2, 0, 0),    // N <= 1024
    MBN_RMS_CFG(1, 4, 4, 0, 0),    // N <= 2048
    MBN_RMS_CFG(4, 2, 2, 0, 8),    // N <= 4096:  512 threads, 2 rows
    MBN_RMS_CFG(8, 1, 2, 0, 0),    // N <= 8192:  512 threads
    MBN_RMS_CFG(2, 2, 16, 2, 4),   // N <= 16384: 256 threads, 2 rows, 2 WGs/CU
    MBN_RMS_CFG(16, 1, 4, 0, 0),   // N <= 32768: 1024 threads
    MBN_RMS_CFG(16, 1, 8, 0, 0),   // N <= 65536: 1024 threads
};

}  // namespace

// Dynamic LDS of a launch: the staged rows, raised to kLdsPerCU / cap when an
// occupancy cap asks for fewer resident workgroups per CU than LDS would allow.
size_t rmsnorm_lds_bytes(int rows, int64_t N, int wgs_per_cu) {
  size_t lds = (size_t)rows * (size_t)N * 2;
  if (wgs_per_cu > 0) {
    const size_t cap = (kLdsPerCU / (size_t)wgs_per_cu) & ~(size_t)511;
    if (cap > lds) lds = cap;
  }
  return lds;
}

hipError_t launch_rmsnorm(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps,
                          hipStream_t stream) {
  const int nchunk = (int)(N / 8);
  const RmsCfg* cfg = nullptr;
  for (const RmsCfg& c : kRmsTable)
    if (nchunk <= c.max_nchunk) { cfg = &c; break; }
  if (!cfg) return hipErrorInvalidValue;
  if (cfg->wpr > 1 && nchunk < 64 * cfg->wpr) return hipErrorInvalidValue;  // table invariant
  const int64_t blocks = (M + cfg->rows - 1) / cfg->rows;
  const size_t lds = rmsnorm_lds_bytes(cfg->rows, N, cfg->wgs_per_cu);
  const float inv_n = 1.0f / (float)N;
  const RmsKernel kernel = (nchunk == cfg->max_nchunk) ? cfg->full : cfg->ragged;
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * cfg->wpr * cfg->rows), lds,
                     stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                     static_cast<uint16_t*>(y), M, nchunk, inv_n, eps, cfg->xcd_group);
  return hipGetLastError();
}

}  // namespace mbn
