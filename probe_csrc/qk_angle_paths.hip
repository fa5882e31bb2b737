// Angle paths of the fused QK-norm + RoPE kernel, for the measurement tools
// (not part of the library): the library's kernel body for one head row per
// wave (few tokens) with the token's sine / cosine obtained in one of three
// ways, each giving the operator's outputs:
//   MODE 0: the library's path: wave 0 forms the 64 angles (one per lane)
//           and shares them through LDS behind a workgroup barrier;
//   MODE 1: every wave forms the 64 angles itself and each lane fetches its 8
//           with ds_bpermute (no LDS table, no barrier);
//   MODE 3: MODE 1 with the rotation products in fp32 instead of fp64.
#include <hip/hip_ext.h>

#include "../memory_bound_normalization_amd/csrc/qk_norm_rope.hip"

namespace mbn {
namespace {

template <typename DT, int MODE>
__global__ void __launch_bounds__(1024)
qkx_kernel(uint16_t* __restrict__ qkv, const uint16_t* __restrict__ q_w, const uint16_t* __restrict__ k_w,
           const int64_t* __restrict__ positions, int n_q, int n_heads, int64_t row_stride, float eps,
           InvFreqPowers inv_pow) {
  __shared__ double2 cs[kHalf];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t token = blockIdx.x;
  const int j = lane & 15;
  uint16_t* const trow = qkv + token * row_stride;
  const int head = wave * kHeadsPerWave + (lane >> 4);
  const int64_t pos_i = positions[token];
  const uint16_t* const qwp = n_q > 0 ? q_w : k_w;
  const uint16_t* const kwp = n_heads > n_q ? k_w : q_w;
  const u32x4 qwv = *reinterpret_cast<const u32x4*>(qwp + 8 * j);
  const u32x4 kwv = *reinterpret_cast<const u32x4*>(kwp + 8 * j);
  const __amdgpu_buffer_rsrc_t heads =
      __builtin_amdgcn_make_buffer_rsrc(trow, (short)0, n_heads * kHeadDim * 2, kBufferWord3);
  const u32x4 xv = __builtin_amdgcn_raw_buffer_load_b128(heads, head * kHeadDim * 2 + 16 * j, 0, kBufferNT);
  asm volatile("" ::"s"(pos_i));

  const bool first_half = j < 8;
  const double sgn = first_half ? -1.0 : 1.0;
  const int i0 = 8 * (first_half ? j : j - 8);
  double hc[8], hs[8];
  if constexpr (MODE == 0) {
    if (wave == 0) {
      const double inv_freq = rope_inv_freq(inv_pow, lane);
      double s, c;
      sincos_reduced((double)pos_i * inv_freq, &s, &c);
      cs[lane] = make_double2(c, s);
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double2 a = cs[i0 + e];
      hc[e] = a.x;
      hs[e] = sgn * a.y;
    }
  } else {
    const double inv_freq = rope_inv_freq(inv_pow, lane);
    double s, c;
    sincos_reduced((double)pos_i * inv_freq, &s, &c);
    const long long cb = __double_as_longlong(c), sb = __double_as_longlong(s);
    const int clo = (int)cb, chi = (int)(cb >> 32), slo = (int)sb, shi = (int)(sb >> 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int src = (i0 + e) << 2;
      const unsigned a0 = (unsigned)__builtin_amdgcn_ds_bpermute(src, clo);
      const unsigned a1 = (unsigned)__builtin_amdgcn_ds_bpermute(src, chi);
      const unsigned b0 = (unsigned)__builtin_amdgcn_ds_bpermute(src, slo);
      const unsigned b1 = (unsigned)__builtin_amdgcn_ds_bpermute(src, shi);
      hc[e] = __longlong_as_double((long long)(((unsigned long long)a1 << 32) | a0));
      hs[e] = sgn * __longlong_as_double((long long)(((unsigned long long)b1 << 32) | b0));
    }
  }
  if (wave * kHeadsPerWave >= n_heads) return;
  const u32x4 wv = head < n_q ? qwv : kwv;
  float x[8], xw[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = DT::lo(xv[e]);
    x[2 * e + 1] = DT::hi(xv[e]);
    xw[2 * e] = x[2 * e] * DT::lo(wv[e]);
    xw[2 * e + 1] = x[2 * e + 1] * DT::hi(wv[e]);
  }
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(x[e], x[e], acc);
  const float ss = row16_sum(acc);
  const float rstd = __builtin_amdgcn_rsqf(__builtin_fmaf(ss, 1.0f / kHeadDim, eps));
  float xwp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) xwp[e] = dpp<kDppRowRor8>(xw[e]);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (MODE == 3) {
      o[e] = __builtin_fmaf(xwp[e], (float)hs[e], xw[e] * (float)hc[e]) * rstd;
    } else {
      const double r = __builtin_fma((double)xwp[e], hs[e], (double)xw[e] * hc[e]);
      o[e] = (float)r * rstd;
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = DT::pack(o[2 * e], o[2 * e + 1]);
  __builtin_amdgcn_raw_buffer_store_b128(out, heads, head * kHeadDim * 2 + 16 * j, 0, kBufferNT);
}

}  // namespace
}  // namespace mbn

// Full rotary, bf16, theta 1e6, eps 1e-6, one step per wave (n_heads <= 64:
// ceil(n_heads / 4) waves per token); the kernel records its own start and end
// in two events. 0 = ok, 1 = invalid arguments, 3 = launch failed.
extern "C" __attribute__((visibility("default"))) int mbn_qk_angle_path(void* qkv, const void* q_w, const void* k_w,
                                                          const int64_t* pos, int64_t T, int hq, int hk, int mode,
                                                          void* stream, void* e0, void* e1) {
  using namespace mbn;
  const int n_heads = hq + hk;
  if (T <= 0 || T > 65536 || n_heads <= 0 || n_heads > 64 || !qkv || !pos || !e0 || !e1) return 1;
  const int waves = (n_heads + 3) / 4;
  const int64_t row_stride = (int64_t)(hq + 2 * hk) * 128;
  const InvFreqPowers ip = rope_inv_freq_powers(1e6f, 128);
  if (mode != 0 && mode != 1 && mode != 3) return 1;
  auto k = mode == 0 ? qkx_kernel<Bf16, 0> : mode == 1 ? qkx_kernel<Bf16, 1> : qkx_kernel<Bf16, 3>;
  hipExtLaunchKernelGGL(k, dim3((unsigned)T), dim3(64 * waves), 0u, (hipStream_t)stream, (hipEvent_t)e0,
                        (hipEvent_t)e1, 0u, static_cast<uint16_t*>(qkv), static_cast<const uint16_t*>(q_w),
                        static_cast<const uint16_t*>(k_w), pos, hq, n_heads, row_stride, 1e-6f, ip);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
