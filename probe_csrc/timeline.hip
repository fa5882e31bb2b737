// Per-workgroup timelines on gfx950, for the measurement tools (not part of
// the library): the library's one-shot row-norm kernel, compiled from its own
// source with its timeline marks defined, and a plain streaming copy with the
// same marks. Each workgroup records the constant-rate wall clock
// (s_memrealtime) at its start, when its data has landed (the row norm: rows
// staged and reduced; the copy: its loads back), after its last store was
// issued and when the workgroup ends, plus the XCD and hardware slot it
// ran on. Thread 0 writes the record with vector stores at the end, so the
// records do not disturb the kernels' per-chunk waits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#define MBN_TL_MAX_BLOCKS (1 << 18)
#define MBN_TL_FIELDS 8

__device__ unsigned long long mbn_tl_trace[MBN_TL_MAX_BLOCKS * MBN_TL_FIELDS];

// s_getreg immediates (size - 1) << 11 | offset << 6 | id: HW_ID (4) and XCC_ID (20).
#define MBN_TL_HWREG(id) ((31 << 11) | (id))

// t2: wave 0 has issued its last store. t3: after a workgroup barrier, every
// wave has issued its last store and the workgroup is about to end (the
// library kernel's waves end right after their stores as well; nothing waits
// for the stores to complete unless MBN_TL_WAIT_STORES is 1, which makes t3
// "every wave's stores completed").
#ifndef MBN_TL_WAIT_STORES
#define MBN_TL_WAIT_STORES 0
#endif
__device__ __forceinline__ void mbn_tl_end(unsigned long long t0, unsigned long long t1) {
  const unsigned long long t2 = __builtin_amdgcn_s_memrealtime();
  if (MBN_TL_WAIT_STORES) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have completed
    __asm__ __volatile__("" ::: "memory");
  }
  __syncthreads();
  const unsigned long long t3 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0 && blockIdx.x < MBN_TL_MAX_BLOCKS) {
    unsigned long long* p = mbn_tl_trace + (size_t)blockIdx.x * MBN_TL_FIELDS;
    p[0] = t0;
    p[1] = t1;
    p[2] = t2;
    p[3] = t3;
    p[4] = (unsigned)__builtin_amdgcn_s_getreg(MBN_TL_HWREG(20));
    p[5] = (unsigned)__builtin_amdgcn_s_getreg(MBN_TL_HWREG(4));
    p[6] = blockIdx.x;
    p[7] = 0x7469'6d65ull;  // record written
  }
}

#define MBN_TL_START() const unsigned long long mbn_tl_t0 = __builtin_amdgcn_s_memrealtime()
#define MBN_TL_LANDED() const unsigned long long mbn_tl_t1 = __builtin_amdgcn_s_memrealtime()
#define MBN_TL_END() mbn_tl_end(mbn_tl_t0, mbn_tl_t1)

#include "../memory_bound_normalization_amd/csrc/rownorm.hip"

namespace mbn {
namespace {

// Wait for every LDS operation of this wave (lgkmcnt(0); vmcnt, expcnt at max).
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __asm__ __volatile__("" ::: "memory");
}

// Pipelined persistent RMSNorm (experiment). A workgroup is one lane set of
// TPR = 64 * WPR lanes; it serves rows g, g + G, g + 2G, ... (G = grid) with
// NB LDS row buffers in a ring: the copies of its first NB rows are issued at
// the start, and as soon as pass 2 of row k has read buffer k % NB (its values
// are in VGPRs, on their way out as stores), the copy of row k + NB is issued
// into it. No workgroup ends before its last row, so no CU slot waits for a
// workgroup's stores to drain and the next one to be dispatched.
//
// Waits: per wave, vector-memory operations complete in issue order. The issue
// order is W (weights), D_0 ... D_{NB-1} (prologue copies), then per row k:
// S_k (its stores), D_{k+NB} (the next copy into the same buffer). When row k
// is taken, the operations issued after chunk q of D_k are D_k's later chunks
// and, for each of the rows k-NB+1 ... k-1, its stores and its refill copy
// (fewer for k < NB-1: only prologue copies and the rows before k). So chunk q
// has landed once at most (MAXC-1-q) + C(k) operations are outstanding, with
// C(k) = (NB-1 + min(k, NB-1)) * MAXC. That holds while every refill up to
// D_{k+NB-1} was issued, i.e. k + NB - 1 < nrows; the last rows wait for
// everything (vmcnt(0)).
template <typename DT, int WPR, int MAXC, int NB>
__global__ void __launch_bounds__(64 * WPR) rms_stream_kernel(RowNormArgs a) {
  constexpr int TPR = 64 * WPR;
  constexpr int NCH = TPR * MAXC;
  static_assert((MAXC - 1) + 2 * (NB - 1) * MAXC <= 63, "vmcnt has 6 bits");
  extern __shared__ u32x4 lds_rows[];  // NB * NCH chunks, then [2][WPR] floats
  float* part = reinterpret_cast<float*>(lds_rows + (size_t)NB * NCH);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t G = gridDim.x;
  const int64_t g = blockIdx.x;
  if (g >= a.M) return;
  const int64_t nrows = (a.M - 1 - g) / G + 1;
  const u32x4* x = reinterpret_cast<const u32x4*>(a.x);
  u32x4* y = reinterpret_cast<u32x4*>(a.y);

  u32x4 wreg[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) wreg[j] = reinterpret_cast<const u32x4*>(a.w)[j * TPR + t];
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  auto copy = [&](int64_t k, int b) {
    const u32x4* xrow = x + (g + k * G) * NCH;
    u32x4* buf = lds_rows + (size_t)b * NCH;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) load_lds_16(xrow + j * TPR + t, (lds_void*)(buf + j * TPR + wave * 64));
  };
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (b < nrows) copy(b, b);

  // C < 0: wait for everything.
  auto row = [&](int64_t k, auto cnt) {
    constexpr int C = decltype(cnt)::value;
    const int b = (int)(k % NB);
    const u32x4* buf = lds_rows + (size_t)b * NCH;
    float acc0 = 0.f, acc1 = 0.f;
    u32x4 first;
    auto take = [&](int j) {
      const u32x4 v = buf[j * TPR + t];
      if (j == 0) first = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = DT::lo(v[e]), q = DT::hi(v[e]);
        acc0 = __builtin_fmaf(p, p, acc0);
        acc1 = __builtin_fmaf(q, q, acc1);
      }
    };
    if constexpr (C < 0) {
      wait_vmem();
#pragma unroll
      for (int j = 0; j < MAXC; ++j) take(j);
    } else {
      static_for<0, MAXC>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        wait_vmcnt_le<MAXC - 1 - Q + C>();
        take(Q);
      });
    }
    float s1[1] = {acc0 + acc1};
    rows_sum<WPR, 1>(s1, nullptr, part + (k & 1) * WPR, NCH, t, wave, 0);
    const float scale = __builtin_amdgcn_rsqf(__builtin_fmaf(s1[0], a.inv_n, a.eps));
    u32x4* yrow = y + (g + k * G) * NCH;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const u32x4 v = (j == 0) ? first : buf[j * TPR + t];
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = DT::pack((DT::lo(v[e]) * scale) * DT::lo(wreg[j][e]), (DT::hi(v[e]) * scale) * DT::hi(wreg[j][e]));
      store_nt_16(yrow + j * TPR + t, o);
    }
    if (k + NB < nrows) {
      wait_lds();  // every LDS read of buffer b has returned (they fed the stores above)
      copy(k + NB, b);
    }
  };

  int64_t k = 0;
  // peeled first rows: fewer operations follow their copies
  static_for<0, NB - 1>([&](auto kk) {
    constexpr int K = decltype(kk)::value;
    if (k < nrows) {
      if (K + NB - 1 < nrows) row(k, std::integral_constant<int, (NB - 1 + K) * MAXC>{});
      else row(k, std::integral_constant<int, -1>{});
      ++k;
    }
  });
  for (; k < nrows; ++k) {
    if (k + NB - 1 < nrows) row(k, std::integral_constant<int, 2 * (NB - 1) * MAXC>{});
    else row(k, std::integral_constant<int, -1>{});
  }
}

}  // namespace
}  // namespace mbn

namespace mbn {
namespace {

__device__ unsigned tl_claim_counter[1];

// One-shot RMSNorm with a claimed tail (experiment): the first `nstatic`
// workgroups each serve their own row block (as the library kernel); the last
// `nclaim` workgroups, dispatched after every static one of their XCD, claim
// the remaining `ndyn` row blocks one at a time from a device counter, so an
// XCD that finishes its static blocks early takes more of the tail. The
// claimer that draws the last failing ticket (ndyn + nclaim - 1) resets the
// counter for the next launch.
template <int WPR, int ROWS, int RPL, int MAXC>
__global__ void __launch_bounds__(64 * WPR * ROWS) tl_claim_kernel(RowNormArgs a, int64_t nstatic, unsigned ndyn,
                                                                   unsigned nclaim) {
  extern __shared__ u32x4 lds_all[];
  const int64_t b = blockIdx.x;
  if (b < nstatic) {
    rownorm_block<Norm::kRms, Bf16, WPR, ROWS, RPL, MAXC, true, true>(a, xcd_remap(b, nstatic, a.xcd_group));
    return;
  }
  int* slot = reinterpret_cast<int*>(lds_all + (size_t)ROWS * RPL * a.nchunk);
  for (;;) {
    __syncthreads();  // the previous block's LDS reads (parked partials included) are done
    if (threadIdx.x == 0) {
      const unsigned tk = atomicAdd(tl_claim_counter, 1u);
      if (tk == ndyn + nclaim - 1) atomicExch(tl_claim_counter, 0u);
      *slot = (int)tk;
    }
    __syncthreads();
    const unsigned tk = (unsigned)*slot;
    if (tk >= ndyn) break;
    rownorm_block<Norm::kRms, Bf16, WPR, ROWS, RPL, MAXC, true, true>(a, nstatic + tk);
  }
}

}  // namespace
}  // namespace mbn

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The streaming copy of stream.hip (lane t owns chunks j * LANES + t, 16-byte
// non-temporal loads and stores) with the marks.
template <int LANES, int CHUNKS>
__global__ void __launch_bounds__(LANES) tl_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  MBN_TL_START();
  const size_t base = (size_t)blockIdx.x * LANES * CHUNKS;
  u32x4 v[CHUNKS];
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) v[j] = __builtin_nontemporal_load(src + base + (size_t)j * LANES + threadIdx.x);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __asm__ __volatile__("" ::: "memory");
  MBN_TL_LANDED();
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j) __builtin_nontemporal_store(v[j], dst + base + (size_t)j * LANES + threadIdx.x);
  MBN_TL_END();
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15) == 0; }

// One-shot RMSNorm kernel of the library's template at a chosen geometry
// (full rows, per-chunk waits): WPR waves per row, ROWS lane sets per
// workgroup, RPL rows per lane set, MAXC chunks per lane; residency cap and
// XCD row group as in the launch tables.
template <int WPR, int ROWS, int RPL, int MAXC>
int tl_variant(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps, hipStream_t s, int cap,
               int group) {
  if (N != (int64_t)64 * WPR * MAXC * 8) return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  a.xcd_group = group;
  const int rows = ROWS * RPL;
  const int64_t blocks = (M + rows - 1) / rows;
  if (blocks * 64 * WPR * ROWS > 0xffffffffLL) return 1;
  const size_t lds = mbn::rownorm_lds_bytes(rows, N, cap);
  hipLaunchKernelGGL((mbn::rownorm_kernel<mbn::Norm::kRms, mbn::Bf16, WPR, ROWS, RPL, MAXC, true, true>),
                     dim3((unsigned)blocks), dim3(64 * WPR * ROWS), lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// The pipelined persistent RMSNorm experiment: variant v selects the
// geometry (waves per row, buffers, workgroups per CU); grid = 256 * per_cu.
template <int WPR, int MAXC, int NB>
int tl_stream(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps, hipStream_t s, int per_cu) {
  if (N != (int64_t)64 * WPR * MAXC * 8) return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  const size_t lds = (size_t)NB * N * 2 + 2 * WPR * sizeof(float);
  const int64_t grid = 256 * (int64_t)per_cu;
  hipLaunchKernelGGL((mbn::rms_stream_kernel<mbn::Bf16, WPR, MAXC, NB>), dim3((unsigned)grid), dim3(64 * WPR), lds, s,
                     a);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Claimed-tail variant at the table's N = 16384 geometry (2 x 128 lanes, one
// row each, cap 2, XCD group 4): ndyn blocks claimed by nclaim workgroups.
int tl_claim(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps, hipStream_t s, unsigned ndyn,
             unsigned nclaim) {
  constexpr int WPR = 2, ROWS = 2, RPL = 1, MAXC = 16;
  if (N != (int64_t)64 * WPR * MAXC * 8 || nclaim == 0) return 1;
  const int rows = ROWS * RPL;
  const int64_t blocks = (M + rows - 1) / rows;
  if ((int64_t)ndyn > blocks) return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.inv_n = 1.0f / (float)N;
  a.eps = eps;
  a.xcd_group = 4;
  size_t lds = mbn::rownorm_lds_bytes(rows, N, 2);
  if (lds < (size_t)rows * N * 2 + 16) lds = (size_t)rows * N * 2 + 16;
  const int64_t nstatic = blocks - ndyn;
  hipLaunchKernelGGL((mbn::tl_claim_kernel<WPR, ROWS, RPL, MAXC>), dim3((unsigned)(nstatic + nclaim)),
                     dim3(64 * WPR * ROWS), lds, s, a, nstatic, ndyn, nclaim);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // namespace

extern "C" {

// RMSNorm through the library's launcher (same tables, same kernels, marks
// compiled in). 0 = ok, 1 = invalid arguments, 3 = launch failed.
__attribute__((visibility("default"))) int mbn_tl_rmsnorm(const void* x, const void* w, void* y, int64_t M,
                                                          int64_t N, float eps, void* stream) {
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || M <= 0 || N <= 0 || N % 8 != 0 || N > 65536 ||
      M > 0x7fffffffLL)
    return 1;
  mbn::RowNormArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.M = M;
  a.nchunk = (int)(N / 8);
  a.eps = eps;
  return mbn::launch_rownorm(mbn::Norm::kRms, mbn::Storage::kBf16, a, (hipStream_t)stream) == hipSuccess ? 0 : 3;
}

// Geometry variants (see tl_variant): 0-9 at N = 16384, 10-19 at N = 32768.
// Returns 1 for an unknown variant or a width it does not fit.
__attribute__((visibility("default"))) int mbn_tl_rmsnorm_variant(const void* x, const void* w, void* y, int64_t M,
                                                                  int64_t N, float eps, void* stream, int v) {
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || M <= 0) return 1;
  const hipStream_t s = (hipStream_t)stream;
  switch (v) {
    case 0: return tl_variant<2, 2, 1, 16>(x, w, y, M, N, eps, s, 2, 4);  // the table's entry
    case 1: return tl_variant<2, 1, 1, 16>(x, w, y, M, N, eps, s, 4, 4);
    case 2: return tl_variant<2, 1, 1, 16>(x, w, y, M, N, eps, s, 2, 4);
    case 3: return tl_variant<4, 1, 1, 8>(x, w, y, M, N, eps, s, 4, 4);
    case 4: return tl_variant<2, 2, 1, 16>(x, w, y, M, N, eps, s, 2, 0);
    case 5: return tl_variant<2, 1, 1, 16>(x, w, y, M, N, eps, s, 5, 4);
    case 6: return tl_variant<2, 2, 1, 16>(x, w, y, M, N, eps, s, 2, 8);
    case 7: return tl_variant<2, 1, 2, 16>(x, w, y, M, N, eps, s, 2, 4);
    case 8: return tl_variant<4, 1, 1, 8>(x, w, y, M, N, eps, s, 3, 4);
    case 9: return tl_variant<2, 2, 1, 16>(x, w, y, M, N, eps, s, 1, 4);
    case 10: return tl_variant<16, 1, 1, 4>(x, w, y, M, N, eps, s, 0, 0);  // the staged-row entry (rows in VGPRs now past 2048 rows)
    case 11: return tl_variant<8, 1, 1, 8>(x, w, y, M, N, eps, s, 2, 0);
    case 12: return tl_variant<4, 1, 1, 16>(x, w, y, M, N, eps, s, 2, 0);
    case 13: return tl_variant<8, 1, 1, 8>(x, w, y, M, N, eps, s, 2, 4);
    case 14: return tl_variant<16, 1, 1, 4>(x, w, y, M, N, eps, s, 0, 4);
    case 15: return tl_variant<4, 1, 1, 16>(x, w, y, M, N, eps, s, 2, 4);
    default: return 1;
  }
}

__attribute__((visibility("default"))) int mbn_tl_rmsnorm_stream(const void* x, const void* w, void* y, int64_t M,
                                                                 int64_t N, float eps, void* stream, int v) {
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || M <= 0) return 1;
  const hipStream_t s = (hipStream_t)stream;
  switch (v) {
    case 0: return tl_stream<2, 16, 2>(x, w, y, M, N, eps, s, 2);   // N = 16384
    case 1: return tl_stream<4, 8, 2>(x, w, y, M, N, eps, s, 2);
    case 2: return tl_stream<4, 8, 3>(x, w, y, M, N, eps, s, 1);
    case 3: return tl_stream<4, 8, 4>(x, w, y, M, N, eps, s, 1);
    case 4: return tl_stream<8, 4, 4>(x, w, y, M, N, eps, s, 1);
    case 5: return tl_stream<2, 16, 2>(x, w, y, M, N, eps, s, 1);
    case 6: return tl_stream<4, 8, 2>(x, w, y, M, N, eps, s, 1);
    case 10: return tl_stream<8, 8, 2>(x, w, y, M, N, eps, s, 1);  // N = 32768
    case 11: return tl_stream<4, 16, 2>(x, w, y, M, N, eps, s, 1);
    case 12: return tl_stream<16, 4, 2>(x, w, y, M, N, eps, s, 1);
    case 20: return tl_stream<2, 8, 2>(x, w, y, M, N, eps, s, 4);  // N = 8192
    case 21: return tl_stream<2, 8, 3>(x, w, y, M, N, eps, s, 3);
    case 22: return tl_stream<1, 16, 2>(x, w, y, M, N, eps, s, 4);
    case 23: return tl_stream<4, 4, 4>(x, w, y, M, N, eps, s, 2);
    default: return 1;
  }
}

__attribute__((visibility("default"))) int mbn_tl_rmsnorm_claim(const void* x, const void* w, void* y, int64_t M,
                                                                int64_t N, float eps, void* stream, unsigned ndyn,
                                                                unsigned nclaim) {
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || M <= 0) return 1;
  return tl_claim(x, w, y, M, N, eps, (hipStream_t)stream, ndyn, nclaim);
}

// Copy of `bytes` (whole workgroups) with 256 lanes x `chunks` (1 or 8) per workgroup.
__attribute__((visibility("default"))) int mbn_tl_copy(const void* src, void* dst, size_t bytes, int chunks,
                                                       void* stream) {
  const size_t per_wg = (size_t)256 * chunks * 16;
  if (!aligned16(src) || !aligned16(dst) || (chunks != 1 && chunks != 8) || bytes == 0 || bytes % per_wg != 0 ||
      bytes / per_wg > 0x7fffffffull)
    return 1;
  const unsigned grid = (unsigned)(bytes / per_wg);
  if (chunks == 1)
    hipLaunchKernelGGL((tl_copy<256, 1>), dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       (u32x4*)dst);
  else
    hipLaunchKernelGGL((tl_copy<256, 8>), dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       (u32x4*)dst);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Zero the records of workgroups [0, nblocks) (host to device copy), or copy
// them to `out` (nblocks * 8 uint64). Synchronous. 0 = ok, 1 = invalid, 3 = HIP error.
__attribute__((visibility("default"))) int mbn_tl_clear(int64_t nblocks) {
  if (nblocks <= 0 || nblocks > MBN_TL_MAX_BLOCKS) return 1;
  const size_t bytes = (size_t)nblocks * MBN_TL_FIELDS * sizeof(unsigned long long);
  void* zero = calloc(1, bytes);
  if (!zero) return 3;
  const hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(mbn_tl_trace), zero, bytes, 0, hipMemcpyHostToDevice);
  free(zero);
  return e == hipSuccess ? 0 : 3;
}

__attribute__((visibility("default"))) int mbn_tl_fetch(unsigned long long* out, int64_t nblocks) {
  if (!out || nblocks <= 0 || nblocks > MBN_TL_MAX_BLOCKS) return 1;
  const size_t bytes = (size_t)nblocks * MBN_TL_FIELDS * sizeof(unsigned long long);
  return hipMemcpyFromSymbol(out, HIP_SYMBOL(mbn_tl_trace), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0 : 3;
}

__attribute__((visibility("default"))) int mbn_tl_max_blocks() { return MBN_TL_MAX_BLOCKS; }

}  // extern "C"
