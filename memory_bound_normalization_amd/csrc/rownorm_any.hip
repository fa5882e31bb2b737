// Row norms of any width: the launch path for rows that are not whole 16-byte
// chunks (N % 8 != 0, which the pages' widening to "non-power-of-two N" in
// "[Inductor] Codegen Gluon", section 3.2, includes) or whose base pointers
// are not 16-byte aligned. Same operations and arithmetic as rownorm.hip
// (RMSNorm, residual add + RMSNorm, LayerNorm, L2Norm; bf16 or fp16 storage).
// Two kernel families, one workgroup per row in both:
//
// rownorm_s16_kernel (with x, y, r and h at one address modulo 16: from
// N = 1024 unless N % 4 == 0 on 8-byte aligned pointers, and from N = 256 on
// pointers that are not 8-byte aligned): the aligned 16-byte
// blocks that cover the row go HBM -> LDS as in the staged-row kernels; the
// neighbouring rows' elements in the two edge blocks are masked out and never
// stored. See the kernel's comment.
//
// rownorm_any_kernel (the other launches): every access is one group of G
// consecutive elements (G = 4, 2 or 1: 8, 4 or 2 bytes), the widest that the
// pointers' alignment allows, and nothing outside a row is read or written.
// With 8-byte aligned pointers and N % 4 != 0 (SHIFT), a row starts mid-group:
// its first 0-3 elements (head) and last 0-3 (tail) are single-element
// accesses by a few lanes, the groups between are 8-byte aligned in x and y,
// and each weight (bias) group is assembled from the two aligned weight groups
// around it, shifted by the head length. 64 * WAVES lanes; lane t owns the
// groups g = j * (64 * WAVES) + t, j < MAXG: they are loaded once into VGPRs
// (all loads of a batch issued before the first use) and the passes run from
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

// Weight (or bias) elements [head + 4 g, head + 4 g + 4) of a vector (8-byte
// aligned) from its aligned 4-element groups g (lo) and g + 1 (hi): lo
// shifted down by `head` elements, filled from hi.
__device__ __forceinline__ u32x2 shift_pair(u32x2 lo, u32x2 hi, int head) {
  if (head == 0) return lo;
  const uint64_t l = __builtin_bit_cast(uint64_t, lo), h = __builtin_bit_cast(uint64_t, hi);
  const int sh = 16 * head;  // 16, 32 or 48
  return __builtin_bit_cast(u32x2, (l >> sh) | (h << (64 - sh)));
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
  constexpr bool kHasW = MODE != Norm::kL2;
  constexpr bool kHasB = MODE == Norm::kLayer;
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
  // Shifted rows: the weight (bias) window of group g spans the vector's
  // aligned groups g and g + 1; the second is clamped to the group that
  // holds element N - 1 (its elements past N - 1 belong to no row element),
  // so both loads are unconditional.
  const int glast = (N - 1) / G;
  for_each([&](greg v, int g) {
    float o[G];
    greg wv{}, bv{};
    if constexpr (SHIFT) {
      const int g1 = g + 1 < glast ? g + 1 : glast;
      if constexpr (kHasW) wv = shift_pair(GR::from(w[g]), GR::from(w[g1]), head);
      if constexpr (kHasB) bv = shift_pair(GR::from(bb[g]), GR::from(bb[g1]), head);
    } else {
      if constexpr (kHasW) wv = GR::from(w[g]);
      if constexpr (kHasB) bv = GR::from(bb[g]);
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

// The 16 bytes at byte offset sh (even, 0 ... 14) of the 32 bytes lo:hi.
template <int Q>
__device__ __forceinline__ u32x4 window_q(u32x4 lo, u32x4 hi, uint32_t r) {
  const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_alignbyte(d[Q + i + 1], d[Q + i], r);
  return o;
}
__device__ __forceinline__ u32x4 window16(u32x4 lo, u32x4 hi, int sh) {
  const uint32_t r = (uint32_t)(sh & 3);
  switch (sh >> 2) {
    case 0: return window_q<0>(lo, hi, r);
    case 1: return window_q<1>(lo, hi, r);
    case 2: return window_q<2>(lo, hi, r);
    default: return window_q<3>(lo, hi, r);
  }
}

// Element e (0 ... 7) of a 16-byte chunk, as raw 16-bit bits.
__device__ __forceinline__ uint32_t chunk_elem(u32x4 v, int e) { return (v[e >> 1] >> (16 * (e & 1))) & 0xffffu; }

// A vector p of N elements (the weight or the bias, 2-byte aligned) on the
// chunk grid of a row whose first element sits h elements into its 16-byte
// block: output chunk k holds row elements [8k - h, 8k - h + 8), whose p
// elements are bytes [sh, sh + 16) of the aligned blocks k and k + 1, counted
// from the block that holds the address of element -h. Both block indices are
// clamped into [b0, b1], the blocks that hold elements of p, so nothing
// outside them is read. Clamping changes only bytes of elements outside
// [0, N), which in the first and last chunk of a row belong to no row element:
// a row element's byte lies in block k or k + 1, and that block holds an
// element of p, hence lies in [b0, b1] and is left unclamped.
struct VecGrid {
  typedef const __attribute__((address_space(1))) u32x4* gvec;
  gvec base;
  int sh, b0, b1;
  __device__ __forceinline__ VecGrid(const uint16_t* p, int h, int N) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(p);
    const uintptr_t a0 = pa - 2 * (uintptr_t)h;
    base = (gvec)(a0 & ~(uintptr_t)15);
    sh = (int)(a0 & 15);
    b0 = (int)((pa >> 4) - (a0 >> 4));
    b1 = (int)(((pa + 2 * (uintptr_t)N - 2) >> 4) - (a0 >> 4));
  }
  // The two blocks of chunk k (the second repeats the first when the window
  // is block-aligned).
  __device__ __forceinline__ void load(int k, u32x4& lo, u32x4& hi) const {
    const int l = k > b0 ? k : b0;
    const int u = sh ? (k + 1 < b1 ? k + 1 : b1) : l;
    lo = base[l];
    hi = base[u];
  }
  __device__ __forceinline__ u32x4 window(u32x4 lo, u32x4 hi) const { return window16(lo, hi, sh); }
};

// Row norms whose rows start anywhere inside a 16-byte block (N % 8 != 0, or
// element-aligned base pointers), with x, y (and r, h) at the same address
// modulo 16. One workgroup per row. The aligned 16-byte chunks that cover the
// row are copied HBM -> LDS as in the staged-row kernels; the first and last
// of them may hold up to 7 elements of the neighbouring rows (same 16-byte
// block, so never another page), which are loaded but masked out of every
// sum and never stored. Compute runs in that chunk grid, which y shares, so
// every interior chunk is one 16-byte store; the two edge chunks store their
// row elements one by one. The weight (bias) chunk of an output chunk starts
// h elements before the chunk (h = the row's offset in its first block): two
// aligned 16-byte loads from L2 (VecGrid), shifted by a byte count that is
// uniform over the row. The loads of all the lane's chunks are issued after
// pass 1, ahead of the reduction, and waited for once before pass 2.
// Workgroup b serves row xcd_remap(b) (runs of xcd_group rows per XCD).
template <Norm MODE, typename DT, int WAVES, int MAXC, bool BATCH>
__global__ void __launch_bounds__(64 * WAVES) rownorm_s16_kernel(RowNormAnyArgs a) {
  constexpr int T = 64 * WAVES;
  constexpr bool kHasR = MODE == Norm::kAddRms;
  __shared__ float part[2][WAVES];
  extern __shared__ u32x4 lds_s16[];  // the row's chunks
  const int N = a.n;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t e0 = xcd_remap(blockIdx.x, gridDim.x, a.xcd_group) * N;  // first element of this row
  const uintptr_t xs = reinterpret_cast<uintptr_t>(a.x + e0);
  const int h = (int)((xs & 15) >> 1);  // elements of the first block before the row
  const int nck = (h + N + 7) >> 3;     // chunks covering the row
  auto chunk_ptr = [&](const uint16_t* base) {
    return reinterpret_cast<const u32x4*>(reinterpret_cast<uintptr_t>(base + e0) - 2 * (uintptr_t)h);
  };
  const u32x4* xc = chunk_ptr(a.x);

#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * T + t;
    if (k < nck) load_lds_16(xc + k, (lds_void*)(lds_s16 + j * T + wave * 64));
  }
  u32x4 rreg[kHasR ? MAXC : 1];
  if constexpr (kHasR) {
    const u32x4* rc = chunk_ptr(a.r);
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * T + t;
      rreg[j] = k < nck ? __builtin_nontemporal_load(rc + k) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  wait_vmem();

  // Element e of chunk k is row element 8k + e - h; a row element iff in [0, N).
  auto in_row = [&](int k, int e) { const int p = 8 * k + e - h; return p >= 0 && p < N; };
  auto is_edge = [&](int k) { return k == 0 || k == nck - 1; };

  // Pass 1 (from LDS): sum of squares (sum for LayerNorm) over the row's
  // elements; the residual add forms h = round(x + r), stores it and
  // continues with the rounded h.
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * T + t;
    if (k < nck) {
      u32x4 v = lds_s16[k];
      const bool edge = is_edge(k);
      if constexpr (kHasR) {
        u32x4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[e] = DT::pack(DT::lo(v[e]) + DT::lo(rreg[j][e]), DT::hi(v[e]) + DT::hi(rreg[j][e]));
        v = hv;
        lds_s16[k] = hv;
        if (edge) {
          for (int e = 0; e < 8; ++e)
            if (in_row(k, e)) __builtin_nontemporal_store((uint16_t)chunk_elem(hv, e), a.h + e0 + 8 * k + e - h);
        } else {
          store_nt_16(const_cast<u32x4*>(chunk_ptr(a.h)) + k, hv);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float val = (e & 1) ? DT::hi(v[e >> 1]) : DT::lo(v[e >> 1]);
        if (edge && !in_row(k, e)) val = 0.f;
        acc = MODE == Norm::kLayer ? acc + val : __builtin_fmaf(val, val, acc);
      }
    }
  }
  // BATCH: the weight (bias) blocks of every chunk of the lane, issued
  // before the reduction (lanes past the row's last chunk load that chunk's
  // blocks); else each chunk's blocks are loaded in pass 2 where it is
  // computed (fewer registers: 8 per chunk and vector).
  constexpr bool kHasW = MODE != Norm::kL2;
  constexpr bool kHasB = MODE == Norm::kLayer;
  constexpr int kHeld = BATCH ? MAXC : 1;
  const VecGrid wg(a.w, h, N), bg(a.b, h, N);
  u32x4 wlo[kHasW ? kHeld : 1], whi[kHasW ? kHeld : 1];
  u32x4 blo[kHasB ? kHeld : 1], bhi[kHasB ? kHeld : 1];
  if constexpr (BATCH) {
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * T + t < nck ? j * T + t : nck - 1;
      if constexpr (kHasW) wg.load(k, wlo[j], whi[j]);
      if constexpr (kHasB) bg.load(k, blo[j], bhi[j]);
    }
  }
  const float s1 = group_sum<WAVES>(acc, part[0], wave);

  float mu = 0.f, scale;
  if constexpr (MODE == Norm::kLayer) {
    mu = s1 * a.inv_n;
    float acc2 = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      const int k = j * T + t;
      if (k < nck) {
        const u32x4 v = lds_s16[k];
        const bool edge = is_edge(k);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float d = ((e & 1) ? DT::hi(v[e >> 1]) : DT::lo(v[e >> 1])) - mu;
          if (edge && !in_row(k, e)) d = 0.f;
          acc2 = __builtin_fmaf(d, d, acc2);
        }
      }
    }
    const float s2 = group_sum<WAVES>(acc2, part[1], wave);
    scale = __builtin_amdgcn_rsqf(s2 * a.inv_n + a.eps);
  } else if constexpr (MODE == Norm::kL2) {
    const float nrm = __builtin_sqrtf(s1);
    scale = 1.0f / ((nrm < a.eps) ? a.eps : nrm);  // NaN norms stay NaN
  } else {
    scale = __builtin_amdgcn_rsqf(__builtin_fmaf(s1, a.inv_n, a.eps));
  }

  u32x4* yc = const_cast<u32x4*>(chunk_ptr(a.y));
  // The batched weight (bias) blocks: one wait here, none between the stores
  // below.
  if constexpr (BATCH) wait_vmem();

  // Pass 2 (from LDS): normalize, weight (and bias), round, store.
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int k = j * T + t;
    if (k < nck) {
      const u32x4 v = lds_s16[k];
      const bool edge = is_edge(k);
      const int64_t p0 = 8 * (int64_t)k - h;
      u32x4 wv{}, bv{};
      if constexpr (!BATCH) {
        if constexpr (kHasW) wg.load(k, wlo[0], whi[0]);
        if constexpr (kHasB) bg.load(k, blo[0], bhi[0]);
      }
      if constexpr (kHasW) wv = wg.window(wlo[BATCH ? j : 0], whi[BATCH ? j : 0]);
      if constexpr (kHasB) bv = bg.window(blo[BATCH ? j : 0], bhi[BATCH ? j : 0]);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = DT::lo(v[e]), q = DT::hi(v[e]);
        if constexpr (MODE == Norm::kLayer) {
          p = __builtin_fmaf((p - mu) * scale, DT::lo(wv[e]), DT::lo(bv[e]));
          q = __builtin_fmaf((q - mu) * scale, DT::hi(wv[e]), DT::hi(bv[e]));
        } else if constexpr (MODE == Norm::kL2) {
          p *= scale;
          q *= scale;
        } else {
          p = (p * scale) * DT::lo(wv[e]);
          q = (q * scale) * DT::hi(wv[e]);
        }
        o[e] = DT::pack(p, q);
      }
      if (edge) {
        for (int e = 0; e < 8; ++e)
          if (in_row(k, e)) __builtin_nontemporal_store((uint16_t)chunk_elem(o, e), a.y + e0 + p0 + e);
      } else {
        store_nt_16(yc + k, o);
      }
    }
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

// The 16-byte staged kernels (rownorm_s16_kernel), by the widest chunk count
// a row of the launch can cover ((N + 14) / 8: up to 7 elements of the
// first block precede the row).
struct S16Cfg {
  int max_nck;
  int waves;
  int xcd_group;
  RowNormAnyKernel k[2];  // [bf16, fp16]
};
#define MBN_S16(MODE, W, C, G, B) \
  S16Cfg { 64 * (W) * (C), W, G, {&rownorm_s16_kernel<MODE, Bf16, W, C, B>, &rownorm_s16_kernel<MODE, F16, W, C, B>} }
// Bands by the widest chunk count of the launch (64 * waves * chunks per
// lane), from a sweep on MI355X of 1-16 waves x 1-8 chunks x XCD runs of 0, 8
// and 16 rows x batched or per-chunk weight loads at N = 511 and 1023
// (element offset 1), 1535, 2047, 3071, 4095, 8191, 16383, 32767 and 65521
// (about 256 MiB per launch): the fastest entry or one within 1.5% of it.
// RMSNorm (also the residual add, and L2Norm, which has no weight):
#define MBN_S16_RMS_BANDS(MODE)                                                                  \
  MBN_S16(MODE, 1, 2, 8, true),       /* N <= 1010:  64 lanes */                                  \
      MBN_S16(MODE, 1, 3, 8, true),   /* N <= 1522 */                                             \
      MBN_S16(MODE, 2, 2, 8, true),   /* N <= 2034:  128 lanes */                                 \
      MBN_S16(MODE, 2, 3, 8, false),  /* N <= 3058 */                                             \
      MBN_S16(MODE, 4, 2, 8, true),   /* N <= 4082:  256 lanes */                                 \
      MBN_S16(MODE, 4, 4, 8, false),  /* N <= 8178 */                                             \
      MBN_S16(MODE, 8, 4, 8, false),  /* N <= 16370: 512 lanes */                                 \
      MBN_S16(MODE, 16, 3, 8, true),  /* N <= 24562: 1024 lanes */                                \
      MBN_S16(MODE, 16, 8, 8, false)  /* N <= 65522 */
const S16Cfg kS16Rms[] = {MBN_S16_RMS_BANDS(Norm::kRms)};
const S16Cfg kS16AddRms[] = {MBN_S16_RMS_BANDS(Norm::kAddRms)};
const S16Cfg kS16L2[] = {MBN_S16_RMS_BANDS(Norm::kL2)};
// LayerNorm (weight and bias: fewer lanes, more chunks per lane, per-chunk
// loads):
const S16Cfg kS16Layer[] = {
    MBN_S16(Norm::kLayer, 1, 2, 0, true),    // N <= 1010:  64 lanes
    MBN_S16(Norm::kLayer, 1, 4, 8, false),   // N <= 2034
    MBN_S16(Norm::kLayer, 1, 8, 8, false),   // N <= 4082
    MBN_S16(Norm::kLayer, 2, 8, 8, false),   // N <= 8178:  128 lanes
    MBN_S16(Norm::kLayer, 4, 8, 8, false),   // N <= 16370: 256 lanes
    MBN_S16(Norm::kLayer, 8, 8, 8, false),   // N <= 32754: 512 lanes
    MBN_S16(Norm::kLayer, 16, 8, 8, false),  // N <= 65522: 1024 lanes
};

template <size_t K>
const S16Cfg* pick_s16(const S16Cfg (&table)[K], int max_nck) {
  for (const S16Cfg& c : table)
    if (max_nck <= c.max_nck) return &c;
  return nullptr;
}
// From kS16MinN on, the staged kernels serve every width except rows of whole
// 4-element groups on 8-byte aligned pointers (N % 4 == 0), where the group
// kernels measured faster (16384 x 16380: 195 against 207 us); from
// kS16MinNarrow they serve only pointers that are not 8-byte aligned (2- and
// 1-element groups otherwise: 65536 x 1001 at an element offset 73 against
// 153 us, 131072 x 511 102 against 154 us, while on 8-byte aligned pointers
// the 4-element groups are faster: 65536 x 1001 64 against 69 us).
constexpr int kS16MinN = 1024;
constexpr int kS16MinNarrow = 256;

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

namespace {

// One launch of the any-width kernels over rows [0, args.M) of args (one
// workgroup per row, at most kMaxWorkItems / 1024 rows).
hipError_t launch_rownorm_any_rows(Norm mode, Storage dtype, RowNormAnyArgs args, hipStream_t stream) {
  const int d = dtype == Storage::kF16 ? 1 : 0;
  // Row tensors at the same address modulo 16 share one chunk grid: the
  // 16-byte staged kernels.
  const uintptr_t m16 = reinterpret_cast<uintptr_t>(args.x) & 15;
  auto same16 = [&](const void* p) { return !p || (reinterpret_cast<uintptr_t>(p) & 15) == m16; };
  const int g4 = rownorm_any_group(args);
  const bool s16 = args.n >= kS16MinN ? !(args.n % 4 == 0 && g4 == 4) : (args.n >= kS16MinNarrow && g4 < 4);
  if (s16 && same16(args.y) && same16(args.r) && same16(args.h)) {
    const int max_nck = (args.n + 14) >> 3;
    const S16Cfg* c = mode == Norm::kLayer    ? pick_s16(kS16Layer, max_nck)
                      : mode == Norm::kAddRms ? pick_s16(kS16AddRms, max_nck)
                      : mode == Norm::kL2     ? pick_s16(kS16L2, max_nck)
                                              : pick_s16(kS16Rms, max_nck);
    if (c) {
      args.xcd_group = c->xcd_group;
      return dispatch(c->k[d], dim3((unsigned)args.M), dim3(64 * c->waves), (size_t)max_nck * 16, stream, args);
    }
  }
  const int g = rownorm_any_group(args);
  const bool shift = g == 4 && args.n % 4 != 0;
  const int groups = (args.n + g - 1) / g;  // shifted rows hold at most N / 4 whole groups
  const AnyCfg* cfg = g == 4 ? pick_any(kAny4, groups) : g == 2 ? pick_any(kAny2, groups) : pick_any(kAny1, groups);
  if (!cfg) return hipErrorInvalidValue;
  const RowNormAnyKernel kernel = cfg->k[shift ? 1 : 0][(int)mode][d];
  const size_t lds = cfg->stage ? (size_t)args.n * 2 : 0;
  return dispatch(kernel, dim3((unsigned)args.M), dim3(64 * cfg->waves), lds, stream, args);
}

}  // namespace

hipError_t launch_rownorm_any(Norm mode, Storage dtype, RowNormAnyArgs args, hipStream_t stream) {
  if (args.n <= 0 || args.M <= 0 || args.M > 0x7fffffffLL) return hipErrorInvalidValue;
  args.inv_n = 1.0f / (float)args.n;
  // One workgroup of at most 1024 lanes per row: beyond kMaxWorkItems / 1024
  // rows the launch runs as several launches over consecutive row ranges (a
  // multiple of 8 rows each, so every range starts at the same address modulo
  // 16 as the tensor and takes the kernel the whole launch would).
  constexpr int64_t kRowsPerLaunch = (kMaxWorkItems / 1024) & ~(int64_t)7;
  for (int64_t r0 = 0; r0 < args.M; r0 += kRowsPerLaunch) {
    RowNormAnyArgs part = args;
    const int64_t e0 = r0 * args.n;
    part.x = args.x + e0;
    part.y = args.y + e0;
    if (args.r) part.r = args.r + e0;
    if (args.h) part.h = args.h + e0;
    part.M = args.M - r0 < kRowsPerLaunch ? args.M - r0 : kRowsPerLaunch;
    const hipError_t err = launch_rownorm_any_rows(mode, dtype, part, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mbn
