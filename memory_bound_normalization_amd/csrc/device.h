// Device helpers shared by the gfx950 kernels: bf16 widening / narrowing,
// 16-lane DPP reductions, and direct HBM->LDS loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mbn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

// bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 values -> two bf16 in one dword (lo in bits 0..15), round to nearest
// even; gfx950 does this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Storage types of 16-bit data: widen either half of a dword to fp32 (exact)
// and narrow two fp32 values to one dword, rounding to nearest even.
struct Bf16 {
  static __device__ __forceinline__ float lo(uint32_t v) { return bf16_lo(v); }
  static __device__ __forceinline__ float hi(uint32_t v) { return bf16_hi(v); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct F16 {
  static __device__ __forceinline__ float lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 f = {a, b};
    f16x2 h = __builtin_convertvector(f, f16x2);
    return __builtin_bit_cast(uint32_t, h);
  }
};

// DPP lane permutations inside a row of 16 lanes.
enum : int {
  kDppQuadXor1 = 0xB1,    // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,    // quad_perm [2,3,0,1]
  kDppRowRor8 = 0x128,    // row_ror:8   (lane j <- lane (j+8) mod 16)
  kDppRowMirror = 0x140,  // lane j <- lane 15-j
  kDppHalfMirror = 0x141, // lane j <- lane 7-j inside each half row
};

template <int Ctrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes. Every lane of the row ends with the same bits:
// each step adds a lane's value and its partner's, and fp32 addition commutes.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}

// Sum over the 64 lanes of a wave, returned in every lane (wave-uniform).
// Fixed order: ((row0 + row1) + (row2 + row3)).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// 16-byte load from global memory straight into LDS (global_load_lds_dwordx4),
// marked non-temporal (the data is read once). Lane l of the wave writes bytes
// [16 l, 16 l + 16) after the wave-uniform LDS address `lds_wave_base`.
// Completion is tracked by vmcnt.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void load_lds_16(const void* gptr, lds_void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_wave_base, 16, 0, kCachePolicyNT);
}

// Wait until every vector-memory load of this wave has landed (LDS included).
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt / lgkmcnt left at max
  __asm__ __volatile__("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt vmcnt(N): vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
  __asm__ __volatile__("" ::: "memory");
}

// f(std::integral_constant<int, I>{}) for I = BEGIN ... END - 1, unrolled at
// compile time (for per-iteration immediates such as wait_vmcnt_le).
template <int BEGIN, int END, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (BEGIN < END) {
    f(std::integral_constant<int, BEGIN>{});
    static_for<BEGIN + 1, END>(f);
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b mod 8). With group = G > 0, XCD x is given runs of G consecutive row
// blocks instead of every 8th one, which changes how the concurrent HBM
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

// Streaming 16-byte store (global_store_dwordx4 ... nt).
__device__ __forceinline__ void store_nt_16(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

}  // namespace mbn
