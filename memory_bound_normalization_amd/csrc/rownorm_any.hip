// Row norms of any width: the launch path for rows that are not whole 16-byte
// chunks (N % 8 != 0, which the pages' widening to "non-power-of-two N" in
// "[Inductor] Codegen Gluon", section 3.2, includes) or whose base pointers
// are not 16-byte aligned. Same operations and arithmetic as rownorm.hip
// (RMSNorm, residual add + RMSNorm, LayerNorm, L2Norm; bf16 or fp16 storage).
// Every access is one group of G consecutive elements (G = 4, 2 or 1: 8, 4 or
// 2 bytes), the widest that the pointers' alignment allows, and nothing
// outside a row is read or written. With 8-byte aligned pointers and N % 4 !=
// 0 (SHIFT), a row starts mid-group: its first 0-3 elements (head) and last
// 0-3 (tail) are single-element accesses by a few lanes, the groups between
// are 8-byte aligned in x and y, and each weight (bias) group is assembled
// from the two aligned weight groups around it, shifted by the head length.
//
// One workgroup per row, 64 * WAVES lanes. Lane t owns the groups
// g = j * (64 * WAVES) + t, j < MAXG: they are loaded once into VGPRs (all
// loads of a batch issued before the first use) and the passes run from
// there, so the row is read from HBM once, as in the method; LDS carries the
// cross-wave partial sums. Rows wider than 32 groups per lane (STAGE) are
// loaded in batches of 32 and kept in LDS for the later passes. Weights and
// bias are group loads that hit L2 after the first rows.
#include "device.h"
#include "kernels.h"

namespace mbn {
namespace {

// A group of G 16-bit elements as it sits in VGPRs, with element access.
template <int G>
struct Grp;
template <>
struct Grp<1> {
  typedef uint16_t mem;  // global memory type of one group
  typedef uint32_t reg;
  static __device__ __forceinline__ reg from(mem m) { return m; }
  static __device__ __forceinline__ mem to(reg r) { return (mem)r; }
  template <typename DT>
  static __device__ __forceinline__ float get(reg r, int) { return DT::lo(r); }
  template <typename DT>
  static __device__ __forceinline__ reg pack(const float (&v)[1]) { return DT::pack(v[0], 0.0f) & 0xffffu; }
};
template <>
struct Grp<2> {
  typedef uint32_t mem;
  typedef uint32_t reg;
  static __device__ __forceinline__ reg from(mem m) { return m; }
  static __device__ __forceinline__ mem to(reg r) { return r; }
  template <typename DT>
  static __device__ __forceinline__ float get(reg r, int i) { return i ? DT::hi(r) : DT::lo(r); }
  template <typename DT>
  static __device__ __forceinline__ reg pack(const float (&v)[2]) { return DT::pack(v[0], v[1]); }
};
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <>
struct Grp<4> {
  typedef u32x2 mem;
  typedef u32x2 reg;
  static __device__ __forceinline__ reg from(mem m) { return m; }
  static __device__ __forceinline__ mem to(reg r) { return r; }
  template <typename DT>
  static __device__ __forceinline__ float get(reg r, int i) {
    const uint32_t d = i < 2 ? r.x : r.y;
    return (i & 1) ? DT::hi(d) : DT::lo(d);
  }
  template <typename DT>
  static __device__ __forceinline__ reg pack(const float (&v)[4]) {
    return reg{DT::pack(v[0], v[1]), DT::pack(v[2], v[3])};
  }
};

// Sum of v over the workgroup (wave64 DPP + readlane, then one LDS step).
template <int WAVES>
__device__ __forceinline__ float group_sum(float v, float* part, int wave) {
  v = wave_sum(v);
  if constexpr (WAVES > 1) {
    if ((threadIdx.x & 63) == 0) part[wave] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) s += part[i];
    v = s;
  }
  return v;
}

// Weight (or bias) elements [head + 4 g, head + 4 g + 4) of the N-element
// vector at p (8-byte aligned) as one group: the aligned group g shifted down
// by `head` elements, filled from group g + 1, whose elements past N (only
// for the last groups) are not read.
__device__ __forceinline__ u32x2 shifted_group(const uint16_t* p, int g, int head, int N) {
  const u32x2* q = reinterpret_cast<const u32x2*>(p);
  if (head == 0) return q[g];
  const uint64_t lo = __builtin_bit_cast(uint64_t, q[g]);
  uint64_t hi = 0;
  if (4 * g + 8 <= N) {
    hi = __builtin_bit_cast(uint64_t, q[g + 1]);
  } else {
    for (int i = 0; i < head; ++i) hi |= (uint64_t)p[4 * g + 4 + i] << (16 * i);
  }
  const int sh = 16 * head;  // 16, 32 or 48
  return __builtin_bit_cast(u32x2, (lo >> sh) | (hi << (64 - sh)));
}

template <Norm MODE, typename DT, int G, int WAVES, int MAXG, bool STAGE, bool SHIFT>
__global__ void __launch_bounds__(64 * WAVES) rownorm_any_kernel(RowNormAnyArgs a) {
  typedef Grp<G> GR;
  typedef typename GR::mem gmem;
  typedef typename GR::reg greg;
  constexpr int T = 64 * WAVES;
  constexpr int BATCH = STAGE ? 32 : MAXG;
  static_assert(MAXG % BATCH == 0, "whole batches");
  static_assert(!STAGE || MAXG > 32, "staged rows are loaded in batches of 32 groups");
  static_assert(!SHIFT || (G == 4 && !STAGE), "shifted rows use 4-element groups in VGPRs");
  __shared__ float part[2][WAVES];  // [reduction][wave]
  extern __shared__ uint32_t lds_any[];  // the row (N / G groups) when STAGE
  gmem* row = reinterpret_cast<gmem*>(lds_any);
  const int N = a.n;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t e0 = (int64_t)blockIdx.x * N;  // first element of this row
  // Groups start `head` elements into the row; `tail` elements follow them.
  int head = 0, ng = N / G, tail = 0;
  if constexpr (SHIFT) {
    head = (int)((4 - (e0 & 3)) & 3);
    if (head > N) head = N;
    ng = (N - head) >> 2;
    tail = N - head - 4 * ng;
  }
  const gmem* x = reinterpret_cast<const gmem*>(a.x + e0 + head);
  const gmem* w = reinterpret_cast<const gmem*>(a.w);
  const gmem* bb = reinterpret_cast<const gmem*>(a.b);
  gmem* y = reinterpret_cast<gmem*>(a.y + e0 + head);

  // SHIFT: lanes t < head + tail each own one head or tail element.
  const bool extra = SHIFT && t < head + tail;
  const int ex = t < head ? t : head + 4 * ng + (t - head);  // its index in the row
  uint32_t xe = 0;
  if (extra) xe = __builtin_nontemporal_load(a.x + e0 + ex);

  // Load (in batches) and pass 1: sum of squares (sum for LayerNorm); the
  // residual add forms h = round(x + r), stores it and continues with the
  // rounded h.
  greg xv[BATCH];
  float acc = 0.f;
#pragma unroll
  for (int b0 = 0; b0 < MAXG; b0 += BATCH) {
#pragma unroll
    for (int jj = 0; jj < BATCH; ++jj) {
      const int g = (b0 + jj) * T + t;
      xv[jj] = g < ng ? GR::from(__builtin_nontemporal_load(x + g)) : greg{};
    }
#pragma unroll
    for (int jj = 0; jj < BATCH; ++jj) {
      const int g = (b0 + jj) * T + t;
      if (g < ng) {
        if constexpr (MODE == Norm::kAddRms) {
          const greg rv = GR::from(__builtin_nontemporal_load(reinterpret_cast<const gmem*>(a.r + e0 + head) + g));
          float hs[G];
#pragma unroll
          for (int i = 0; i < G; ++i)
            hs[i] = GR::template get<DT>(xv[jj], i) + GR::template get<DT>(rv, i);
          xv[jj] = GR::template pack<DT>(hs);
          __builtin_nontemporal_store(GR::to(xv[jj]), reinterpret_cast<gmem*>(a.h + e0 + head) + g);
        }
        if constexpr (STAGE) row[g] = GR::to(xv[jj]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const float v = GR::template get<DT>(xv[jj], i);
          acc = MODE == Norm::kLayer ? acc + v : __builtin_fmaf(v, v, acc);
        }
      }
    }
  }
  if (extra) {
    float v = DT::lo(xe);
    if constexpr (MODE == Norm::kAddRms) {
      xe = DT::pack(v + DT::lo(__builtin_nontemporal_load(a.r + e0 + ex)), 0.0f) & 0xffffu;
      __builtin_nontemporal_store((uint16_t)xe, a.h + e0 + ex);
      v = DT::lo(xe);
    }
    acc = MODE == Norm::kLayer ? acc + v : __builtin_fmaf(v, v, acc);
  }
  const float s1 = group_sum<WAVES>(acc, part[0], wave);

  // The later passes visit this lane's groups (value, index) in order: from
  // VGPRs, or from LDS when STAGE (each lane reads back only what it wrote,
  // so LDS needs no barrier).
  auto for_each = [&](auto&& f) {
    if constexpr (STAGE) {
#pragma unroll 4
      for (int g = t; g < ng; g += T) f(GR::from(row[g]), g);
    } else {
#pragma unroll
      for (int j = 0; j < MAXG; ++j)
        if (j * T + t < ng) f(xv[j], j * T + t);
    }
  };

  float mu = 0.f, scale;
  if constexpr (MODE == Norm::kLayer) {
    mu = s1 * a.inv_n;
    float acc2 = 0.f;
    for_each([&](greg v, int) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float d = GR::template get<DT>(v, i) - mu;
        acc2 = __builtin_fmaf(d, d, acc2);
      }
    });
    if (extra) {
      const float d = DT::lo(xe) - mu;
      acc2 = __builtin_fmaf(d, d, acc2);
    }
    const float s2 = group_sum<WAVES>(acc2, part[1], wave);
    scale = __builtin_amdgcn_rsqf(s2 * a.inv_n + a.eps);
  } else if constexpr (MODE == Norm::kL2) {
    const float nrm = __builtin_sqrtf(s1);
    scale = 1.0f / ((nrm < a.eps) ? a.eps : nrm);  // NaN norms stay NaN
  } else {
    scale = __builtin_amdgcn_rsqf(__builtin_fmaf(s1, a.inv_n, a.eps));
  }

  // Pass 2: normalize, weight (and bias), round, store.
  auto out1 = [&](float p, float wv, float bv) -> float {
    if constexpr (MODE == Norm::kLayer) return __builtin_fmaf((p - mu) * scale, wv, bv);
    else if constexpr (MODE == Norm::kL2) return p * scale;
    else return (p * scale) * wv;
  };
  for_each([&](greg v, int g) {
    float o[G];
    greg wv{}, bv{};
    if constexpr (SHIFT) {
      if constexpr (MODE != Norm::kL2) wv = shifted_group(a.w, g, head, N);
      if constexpr (MODE == Norm::kLayer) bv = shifted_group(a.b, g, head, N);
    } else {
      if constexpr (MODE != Norm::kL2) wv = GR::from(w[g]);
      if constexpr (MODE == Norm::kLayer) bv = GR::from(bb[g]);
    }
#pragma unroll
    for (int i = 0; i < G; ++i)
      o[i] = out1(GR::template get<DT>(v, i), GR::template get<DT>(wv, i), GR::template get<DT>(bv, i));
    __builtin_nontemporal_store(GR::to(GR::template pack<DT>(o)), y + g);
  });
  if (extra) {
    const float wv = MODE != Norm::kL2 ? DT::lo(a.w[ex]) : 0.f;
    const float bv = MODE == Norm::kLayer ? DT::lo(a.b[ex]) : 0.f;
    __builtin_nontemporal_store((uint16_t)(DT::pack(out1(DT::lo(xe), wv, bv), 0.0f) & 0xffffu), a.y + e0 + ex);
  }
}

typedef void (*RowNormAnyKernel)(RowNormAnyArgs);

// One band of widths: groups per lane and lanes per row for each group size.
struct AnyCfg {
  int max_groups;  // widest row served, in groups
  int waves;
  bool stage;      // row kept in LDS (N * 2 bytes of dynamic LDS)
  RowNormAnyKernel k[2][4][2];  // [shifted][mode][bf16, fp16]
};

#define MBN_ANY_MODE(MODE, G, W, E, S, SH) \
  { &rownorm_any_kernel<MODE, Bf16, G, W, E, S, SH>, &rownorm_any_kernel<MODE, F16, G, W, E, S, SH> }
#define MBN_ANY_MODES(G, W, E, S, SH)                                                          \
  {                                                                                            \
    MBN_ANY_MODE(Norm::kRms, G, W, E, S, SH), MBN_ANY_MODE(Norm::kAddRms, G, W, E, S, SH),     \
        MBN_ANY_MODE(Norm::kLayer, G, W, E, S, SH), MBN_ANY_MODE(Norm::kL2, G, W, E, S, SH)    \
  }
// Bands of G = 1 and 2 (no shifted variant: the slot repeats the plain one).
#define MBN_ANY_CFG(G, W, E, S) \
  AnyCfg { 64 * (W) * (E), W, S, {MBN_ANY_MODES(G, W, E, S, false), MBN_ANY_MODES(G, W, E, S, false)} }
// Bands of G = 4, with the shifted variant for N % 4 != 0.
#define MBN_ANY_CFG4(W, E) \
  AnyCfg { 64 * (W) * (E), W, false, {MBN_ANY_MODES(4, W, E, false, false), MBN_ANY_MODES(4, W, E, false, true)} }

// Bands per group size, narrowest first: at most 32 VGPRs of row data per
// lane (64 elements for G = 2 and 4, 32 for G = 1); the widest G = 1 rows are
// staged in LDS instead.
const AnyCfg kAny1[] = {
    MBN_ANY_CFG(1, 1, 8, false),    // N <= 512:   64 lanes
    MBN_ANY_CFG(1, 4, 8, false),    // N <= 2048:  256 lanes
    MBN_ANY_CFG(1, 4, 32, false),   // N <= 8192
    MBN_ANY_CFG(1, 16, 32, false),  // N <= 32768: 1024 lanes
    MBN_ANY_CFG(1, 16, 64, true),   // N <= 65536: row in LDS
};
const AnyCfg kAny2[] = {
    MBN_ANY_CFG(2, 1, 8, false),    // N <= 1024:  64 lanes
    MBN_ANY_CFG(2, 4, 8, false),    // N <= 4096:  256 lanes
    MBN_ANY_CFG(2, 4, 16, false),   // N <= 8192
    MBN_ANY_CFG(2, 16, 16, false),  // N <= 32768: 1024 lanes
    MBN_ANY_CFG(2, 16, 32, false),  // N <= 65536
};
const AnyCfg kAny4[] = {
    MBN_ANY_CFG4(1, 4),    // N <= 1024:  64 lanes
    MBN_ANY_CFG4(4, 4),    // N <= 4096:  256 lanes
    MBN_ANY_CFG4(4, 8),    // N <= 8192
    MBN_ANY_CFG4(16, 8),   // N <= 32768: 1024 lanes
    MBN_ANY_CFG4(16, 16),  // N <= 65536
};

template <size_t K>
const AnyCfg* pick_any(const AnyCfg (&table)[K], int groups) {
  for (const AnyCfg& c : table)
    if (groups <= c.max_groups) return &c;
  return nullptr;
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

int rownorm_any_group(const RowNormAnyArgs& a) {
  auto all_aligned = [&](uintptr_t al) {
    return aligned_to(a.x, al) && aligned_to(a.r, al) && aligned_to(a.w, al) && aligned_to(a.b, al) &&
           aligned_to(a.h, al) && aligned_to(a.y, al);
  };
  if (all_aligned(8)) return 4;  // N % 4 != 0: shifted groups
  if (a.n % 2 == 0 && all_aligned(4)) return 2;
  return 1;
}

hipError_t launch_rownorm_any(Norm mode, Storage dtype, RowNormAnyArgs args, hipStream_t stream) {
  if (args.n <= 0 || args.M <= 0 || args.M > 0x7fffffffLL) return hipErrorInvalidValue;
  const int g = rownorm_any_group(args);
  const bool shift = g == 4 && args.n % 4 != 0;
  const int groups = (args.n + g - 1) / g;  // shifted rows hold at most N / 4 whole groups
  const AnyCfg* cfg = g == 4 ? pick_any(kAny4, groups) : g == 2 ? pick_any(kAny2, groups) : pick_any(kAny1, groups);
  if (!cfg) return hipErrorInvalidValue;
  args.inv_n = 1.0f / (float)args.n;
  const RowNormAnyKernel kernel = cfg->k[shift ? 1 : 0][(int)mode][dtype == Storage::kF16 ? 1 : 0];
  const size_t lds = cfg->stage ? (size_t)args.n * 2 : 0;
  hipLaunchKernelGGL(kernel, dim3((unsigned)args.M), dim3(64 * cfg->waves), lds, stream, args);
  return hipGetLastError();
}

}  // namespace mbn
