// Fused per-head QK RMSNorm + rotary embedding (rotate-half pairing), in place
// on a packed QKV tensor, for gfx950.
//
// Dataflow from "[pretuned] Optimize fused_qk_norm_rope on B200", Summary (full
// rotary case): both rotary halves of a head are loaded once, the head's RMS is
// reduced from those register-resident values, the Q/K weight and the rotation
// are applied with no trip through memory, and each half is stored once. There
// is no store followed by a reload, hence no barrier between them.
//
// Mapping: one workgroup per token. A head of 128 bf16 is 16 lanes x 16
// bytes, i.e. one DPP row, so a wave holds 4 heads, the head's sum of squares
// is a 16-lane DPP reduction and the rotary partner of lane j (the chunk 64
// elements away) is lane j ^ 8 of the same row, fetched with row_ror:8.
// The inverse frequencies theta^(-2i/R) do not depend on the token. The host
// evaluates the six powers theta^(-2^(k+1)/R) once per launch in fp64 and
// passes them as kernel arguments; lane i forms theta^(-2i/R) as the product
// of the powers whose bit k is set in i. Those are uniform (scalar) loads, so
// the angle work does not wait for the head loads issued before it.
// Wave 0 forms the token's 64 angles pos * inv_freq and their sin / cos in
// fp64 (one per lane, sincos_reduced) once and shares cos / sin through 1 KiB
// of LDS; the
// waves then step over the token's heads 4 at a time. Few tokens: one wave
// per 4 heads (a single step, lowest latency); up to 1024 tokens half as many
// waves, two steps each. Many tokens: 4 waves per token, looping, so the
// per-token angle work is not repeated in every wave.
//
// Each wave issues the loads of a group of up to KMAX of its steps before the
// arithmetic of the first (the first group's before the angle work), so KMAX
// head rows per wave are in flight: KMAX = 3 with 4 waves per token (all of a
// wave's steps for up to 48 heads), 2 with two steps per wave, else 1; with
// KMAX > 1 the lane's cos / sin stay in registers across the steps. The
// token's q and k heads are addressed through a buffer resource that ends at
// the last head: lanes past it (head counts not a multiple of 4, steps past a
// wave's last) load zeros and their stores are dropped by the hardware's
// range check, so every load and store is unconditional and the compiler's
// wait before a step covers that step's row only. The head rows are read
// once and written once: their loads and stores are non-temporal.
//
// Partial rotary (rotary_dim R < 128, a multiple of 16; the page keeps the
// full-head norm for it since the tail must still be normalized): the RMS and
// the weight cover the whole head, chunks [0, R/8) rotate with the partner
// chunk R/16 away (fetched with ds_bpermute instead of row_ror:8) and angles
// pos * theta^(-2i/R), and chunks [R/8, 16) are stored normalized only.
//
// Precision: x * w is exact in fp32 (two 8-bit significands for bf16, two
// 11-bit ones for fp16). The rotation
// x*w*cos -/+ x'*w'*sin is formed in fp64 because outputs of near-cancelling
// pairs are judged on an absolute floor of about 1e-6, which fp32 products of
// magnitude ~7 would consume on their own; rstd only scales the result
// (relative error), so it stays fp32.
#include <cmath>

#include "device.h"
#include "kernels.h"
#include "rope_math.h"

namespace mbn {
namespace {

constexpr int kHeadDim = 128;
constexpr int kHalf = kHeadDim / 2;
constexpr int kHeadsPerWave = 4;

// Cache-policy bits of a buffer access: non-temporal.
constexpr int kBufferNT = 2;
// Word 3 of a raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;

template <typename DT, int KMAX>
__global__ void __launch_bounds__(1024)
qk_norm_rope_kernel(uint16_t* __restrict__ qkv, const uint16_t* __restrict__ q_w,
                    const uint16_t* __restrict__ k_w, const int64_t* __restrict__ positions,
                    int n_q, int n_heads, int64_t row_stride, int rot_chunks, float eps,
                    InvFreqPowers inv_pow) {
  __shared__ double2 cs[kHalf];  // (cos, sin) of the token's rot_chunks * 8 angles

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int64_t token = blockIdx.x;
  const int j = lane & 15;  // 16-byte chunk of the head: elements [8j, 8j + 8)
  uint16_t* const trow = qkv + token * row_stride;
  // Step s of this wave covers heads wave0 + s * step_heads + [0, 4); lane
  // row r = lane >> 4 takes head wave0 + s * step_heads + r.
  const int wave0 = wave * kHeadsPerWave;
  const int step_heads = waves * kHeadsPerWave;

  // The token's position: a uniform (scalar) load, issued with the head loads
  // and kept there (see below) rather than moved into wave 0's angle branch
  // behind further argument loads.
  const int64_t pos_i = positions[token];
  // Both weight chunks of the lane, loaded ahead of the head rows so that
  // waiting for them never waits for a head row. A weight with no heads may be
  // null: its chunk is then read from the other weight and never used.
  const uint16_t* const qwp = n_q > 0 ? q_w : k_w;
  const uint16_t* const kwp = n_heads > n_q ? k_w : q_w;
  const u32x4 qwv = *reinterpret_cast<const u32x4*>(qwp + 8 * j);
  const u32x4 kwv = *reinterpret_cast<const u32x4*>(kwp + 8 * j);
  // The token's q and k heads, n_heads * 256 bytes: accesses at or past the
  // end read zeros or write nothing.
  const __amdgpu_buffer_rsrc_t heads =
      __builtin_amdgcn_make_buffer_rsrc(trow, (short)0, n_heads * kHeadDim * 2, kBufferWord3);
  // Loads of steps s0 ... s0 + KMAX - 1, issued before the angle computation
  // (first group) or the group's arithmetic.
  u32x4 xs[KMAX];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      const int head = wave0 + (s0 + s) * step_heads + (lane >> 4);
      xs[s] = __builtin_amdgcn_raw_buffer_load_b128(heads, head * kHeadDim * 2 + 16 * j, 0, kBufferNT);
    }
  };
  load_group(0);

  // Using the position here keeps its load ahead of this point; the wait
  // counts scalar loads only, so the head loads stay in flight.
  asm volatile("" ::"s"(pos_i));
  // Angle i = lane: phi = pos * theta^(-2i/R), fp64, R = rotary dimension.
  const int half = 8 * rot_chunks;  // R / 2
  if (wave == 0 && lane < half) {
    const double inv_freq = rope_inv_freq(inv_pow, lane);
    const double pos = (double)pos_i;
    double s, c;
    sincos_reduced(pos * inv_freq, &s, &c);
    cs[lane] = make_double2(c, s);
  }
  __syncthreads();

  // Chunk j < rot_chunks pairs with j + rot_chunks (sign -), chunk j in
  // [rot_chunks, 2 rot_chunks) with j - rot_chunks (sign +); later chunks are
  // not rotated.
  const bool full = rot_chunks == 8;
  const bool rotated = j < 2 * rot_chunks;
  const bool first_half = j < rot_chunks;
  const double sgn = first_half ? -1.0 : 1.0;
  const int i0 = 8 * (first_half ? j : j - rot_chunks);
  const int partner = (lane & ~15) | (rotated ? (first_half ? j + rot_chunks : j - rot_chunks) : j);
  // With several steps per group the lane's 8 (cos, +/-sin) pairs stay in
  // registers; a single step reads them from LDS where they are used (fewer
  // registers, more waves resident).
  constexpr bool kHoist = KMAX > 1;
  double hc[kHoist ? 8 : 1], hs[kHoist ? 8 : 1];
  if constexpr (kHoist) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double2 a = rotated ? cs[i0 + e] : make_double2(1.0, 0.0);
      hc[e] = a.x;
      hs[e] = sgn * a.y;
    }
  }
  // Every lane of a wave runs the same steps (the DPP exchanges need the
  // whole row of 16 lanes): a step runs while the wave's first head in it
  // exists.
  for (int s0 = 0;; s0 += KMAX) {
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      const int base = wave0 + (s0 + s) * step_heads;
      if (base >= n_heads) return;
      const int head = base + (lane >> 4);
      const u32x4 xv = xs[s];
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

      float xwp[8];  // partner chunk (R/2 elements away), same head
      if (full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xwp[e] = dpp<kDppRowRor8>(xw[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xwp[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(partner << 2, __float_as_int(xw[e])));
      }

      // first half: o_i = u_i cos - u_{i+R/2} sin; second half: o = u cos + u_{i-R/2} sin
      float o[8];
      if (rotated) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          double r;
          if constexpr (kHoist) {
            r = __builtin_fma((double)xwp[e], hs[e], (double)xw[e] * hc[e]);
          } else {
            const double2 a = cs[i0 + e];
            r = __builtin_fma((double)xwp[e], sgn * a.y, (double)xw[e] * a.x);
          }
          o[e] = (float)r * rstd;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = xw[e] * rstd;
      }
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = DT::pack(o[2 * e], o[2 * e + 1]);
      __builtin_amdgcn_raw_buffer_store_b128(out, heads, head * kHeadDim * 2 + 16 * j, 0, kBufferNT);
    }
    if (wave0 + (s0 + KMAX) * step_heads >= n_heads) return;
    load_group(s0 + KMAX);
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(Storage dtype, void* qkv, const void* q_w, const void* k_w,
                               const int64_t* positions, int64_t T, int n_q_heads,
                               int n_kv_heads, int rotary_dim, float eps, float theta,
                               hipStream_t stream) {
  const int n_heads = n_q_heads + n_kv_heads;
  const int groups = (n_heads + kHeadsPerWave - 1) / kHeadsPerWave;
  // Up to 512 tokens: one wave per 4-head group (at most 16 waves, a single
  // step); up to 1024, half as many waves (two steps); beyond, 4 waves per
  // token. Chosen on MI355X for 32 q + 8 k heads: back to back, T = 256 3.4 us
  // with 10 waves against 4.1 us with 4; per launch, T = 1024 6.0 us with 5
  // waves against 6.6 us with 4, T = 4096 16.3 us with 4 waves against 17.1
  // with 5 and 17.0 with 2, T = 65536 217 us with 4 against 224 with 5 and 222
  // with 2.
  const int all = groups < 16 ? groups : 16;
  const int waves = T <= 512 ? all : T <= 1024 ? (all + 1) / 2 : (groups < 4 ? groups : 4);
  const int64_t row_stride = (int64_t)(n_q_heads + 2 * n_kv_heads) * kHeadDim;
  // The inverse frequency of pair i is theta^(-2i/R) = prod over the set bits
  // k of i of theta^(-2^(k+1)/R): six fp64 pows on the host (the C library's
  // pow, within an ulp each), at most six fp64 products on the device, so a
  // relative error of about 1e-15 (an angle error of 1e-15 * phi rad).
  const InvFreqPowers inv_pow = rope_inv_freq_powers(theta, rotary_dim);
  // Head rows in flight per wave (KMAX): all of a wave's steps, at most 3.
  // Measured on MI355X for 32 q + 8 k heads, per launch, against one row in
  // flight: 65536 tokens 215 us against 223, 16384 54.2 us against 58.5, 4096
  // 16.3 us against 17.6, 1024 6.0 us against 6.7, 768 5.0 us against 6.0.
  const int steps = (groups + waves - 1) / waves;
  const int kmax = steps < 3 ? steps : 3;
  const auto kernel =
      dtype == Storage::kF16
          ? (kmax == 3 ? qk_norm_rope_kernel<F16, 3> : kmax == 2 ? qk_norm_rope_kernel<F16, 2> : qk_norm_rope_kernel<F16, 1>)
          : (kmax == 3 ? qk_norm_rope_kernel<Bf16, 3> : kmax == 2 ? qk_norm_rope_kernel<Bf16, 2> : qk_norm_rope_kernel<Bf16, 1>);
  // One workgroup per token; beyond kMaxWorkItems work-items, several launches
  // over consecutive token ranges.
  const int64_t tokens_per_launch = kMaxWorkItems / (64 * waves);
  for (int64_t t0 = 0; t0 < T; t0 += tokens_per_launch) {
    const int64_t nt = T - t0 < tokens_per_launch ? T - t0 : tokens_per_launch;
    const hipError_t err =
        dispatch(kernel, dim3((unsigned)nt), dim3(64 * waves), 0, stream,
                 static_cast<uint16_t*>(qkv) + t0 * row_stride, static_cast<const uint16_t*>(q_w),
                 static_cast<const uint16_t*>(k_w), positions + t0, n_q_heads, n_heads, row_stride,
                 rotary_dim / 16, eps, inv_pow);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace mbn
