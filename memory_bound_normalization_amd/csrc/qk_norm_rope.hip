// Fused per-head QK RMSNorm + rotary embedding (rotate-half pairing), in place
// on a packed QKV tensor, for gfx950.
//
// Dataflow from "[pretuned] Optimize fused_qk_norm_rope on B200", Summary (full
// rotary case): both rotary halves of a head are loaded once, the head's RMS is
// reduced from those register-resident values, the Q/K weight and the rotation
// are applied with no trip through memory, and each half is stored once. There
// is no store followed by a reload, hence no barrier between them.
//
// Mapping: one wave per (token, group of 4 heads). A head of 128 bf16 is 16
// lanes x 16 bytes, i.e. one DPP row, so the head's sum of squares is a
// 16-lane DPP reduction and the rotary partner of lane j (the chunk 64
// elements away) is lane j ^ 8 of the same row, fetched with row_ror:8.
// The wave first evaluates the token's 64 angles in fp64 (one per lane) and
// shares cos / sin through 1 KiB of LDS.
//
// Precision: x * w is exact in fp32 (two 8-bit significands). The rotation
// x*w*cos -/+ x'*w'*sin is formed in fp64 because outputs of near-cancelling
// pairs are judged on an absolute floor of about 1e-6, which fp32 products of
// magnitude ~7 would consume on their own; rstd only scales the result
// (relative error), so it stays fp32.
#include "device.h"
#include "kernels.h"

namespace mbn {
namespace {

constexpr int kHeadDim = 128;
constexpr int kHalf = kHeadDim / 2;
constexpr int kHeadsPerWave = 4;

__global__ void __launch_bounds__(64)
qk_norm_rope_kernel(uint16_t* __restrict__ qkv, const uint16_t* __restrict__ q_w,
                    const uint16_t* __restrict__ k_w, const int64_t* __restrict__ positions,
                    int n_q, int n_heads, int groups, int64_t row_stride, float eps,
                    double theta) {
  __shared__ double2 cs[kHalf];  // (cos, sin) of the token's 64 angles

  const int lane = threadIdx.x;
  const int64_t token = blockIdx.x / groups;
  const int group = (int)(blockIdx.x - token * groups);
  const int head = group * kHeadsPerWave + (lane >> 4);
  const int j = lane & 15;  // 16-byte chunk of the head: elements [8j, 8j + 8)
  const bool live = head < n_heads;

  // Issue the head load first so it overlaps the angle computation.
  uint16_t* hp = qkv + token * row_stride + (int64_t)head * kHeadDim + 8 * j;
  const uint16_t* wp = (head < n_q ? q_w : k_w) + 8 * j;
  u32x4 xv = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
  if (live) {
    xv = *reinterpret_cast<const u32x4*>(hp);
    wv = *reinterpret_cast<const u32x4*>(wp);
  }

  // Angle i = lane: phi = pos * theta^(-2i/D), fp64.
  {
    const double pos = (double)positions[token];
    const double inv_freq = pow(theta, -(double)(2 * lane) / (double)kHeadDim);
    double s, c;
    sincos(pos * inv_freq, &s, &c);
    cs[lane] = make_double2(c, s);
  }
  __syncthreads();

  float x[8], xw[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(xv[e]);
    x[2 * e + 1] = bf16_hi(xv[e]);
    xw[2 * e] = x[2 * e] * bf16_lo(wv[e]);
    xw[2 * e + 1] = x[2 * e + 1] * bf16_hi(wv[e]);
  }
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(x[e], x[e], acc);
  const float ss = row16_sum(acc);
  const float rstd = __builtin_amdgcn_rsqf(__builtin_fmaf(ss, 1.0f / kHeadDim, eps));

  float xwp[8];  // partner chunk (64 elements away), same head
#pragma unroll
  for (int e = 0; e < 8; ++e) xwp[e] = dpp<kDppRowRor8>(xw[e]);

  // first half: o_i = u_i cos - u_{i+64} sin; second half: o = u cos + u_{i-64} sin
  const double sgn = (j < 8) ? -1.0 : 1.0;
  const int i0 = 8 * (j & 7);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double2 a = cs[i0 + e];
    const double r = __builtin_fma((double)xwp[e], sgn * a.y, (double)xw[e] * a.x);
    o[e] = (float)r * rstd;
  }
  if (live) {
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
    *reinterpret_cast<u32x4*>(hp) = out;
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(void* qkv, const void* q_w, const void* k_w,
                               const int64_t* positions, int64_t T, int n_q_heads,
                               int n_kv_heads, float eps, float theta, hipStream_t stream) {
  const int n_heads = n_q_heads + n_kv_heads;
  const int groups = (n_heads + kHeadsPerWave - 1) / kHeadsPerWave;
  const int64_t blocks = T * groups;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t row_stride = (int64_t)(n_q_heads + 2 * n_kv_heads) * kHeadDim;
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)blocks), dim3(64), 0, stream,
                     static_cast<uint16_t*>(qkv), static_cast<const uint16_t*>(q_w),
                     static_cast<const uint16_t*>(k_w), positions, n_q_heads, n_heads, groups,
                     row_stride, eps, (double)theta);
  return hipGetLastError();
}

}  // namespace mbn
