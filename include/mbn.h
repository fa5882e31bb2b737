/*
 * mbn.h -- C interface of the memory-bound normalization library (libmbn.so),
 * MI355X / gfx950.
 *
 * Conventions shared by every entry point:
 *   - Tensors are raw device pointers owned by the caller. bf16 means the raw
 *     16-bit IEEE bfloat16 bit pattern. Arrays are row-major and contiguous.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *     is enqueued on it asynchronously; the library never synchronizes,
 *     never allocates device or host memory and issues nothing but kernel
 *     launches, so its calls may be captured into a HIP graph.
 *   - Every argument is validated on the host before any HIP call. A non-zero
 *     status means nothing was launched (except MBN_EHIP, which reports that
 *     the launch itself failed; the HIP error state is read and cleared with
 *     hipGetLastError).
 *   - The library keeps no state between calls and may be called from several
 *     host threads.
 *   - Results are deterministic: a fixed reduction order, no atomics.
 */
#ifndef MBN_H
#define MBN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MBN_API __attribute__((visibility("default")))

/* Status codes returned by every entry point. */
#define MBN_OK 0           /* success (also for empty inputs: nothing launched) */
#define MBN_EINVAL 1       /* an argument is invalid: null pointer, negative size,
                              eps negative / NaN / infinite, odd head_dim,
                              overlapping input and output ranges */
#define MBN_EUNSUPPORTED 2 /* valid but outside what the kernels handle: row
                              wider than MBN_RMSNORM_MAX_N, a row-norm pointer
                              at an odd address, a QK pointer not 16-byte
                              aligned, head_dim other than MBN_QK_HEAD_DIM */
#define MBN_EHIP 3         /* the kernel launch failed */

/* Widest row of the row norms: one row is staged whole in LDS (2 bytes per
 * element). */
#define MBN_RMSNORM_MAX_N 65536
/* Head size handled by qk_norm_rope_fwd. */
#define MBN_QK_HEAD_DIM 128

/*
 * rmsnorm_fwd -- row-wise RMSNorm forward in bf16.
 *
 * Defined by "[Inductor] Codegen Gluon", section 3.1 (the RMSNorm reference
 * workload: x is read for the x*x accumulation and again for x * rstd *
 * weight). For every row i of x:
 *     rstd_i = 1 / sqrt( (1/N) * sum_j x[i,j]^2 + eps )
 *     y[i,j] = bf16( x[i,j] * rstd_i * w[j] )
 * Each row is read from HBM once and staged in LDS as bf16; both the sum of
 * squares and the scaling read the staged copy and widen to fp32 there. The
 * sum of squares and the products are fp32; the output is rounded to nearest
 * even.
 *
 *   x      device, bf16 [M, N], read only (unless y == x)
 *   w      device, bf16 [N], read only
 *   y      device, bf16 [M, N], written. y == x (exact alias, in place) is
 *          allowed; any other overlap of y with x or w is MBN_EINVAL.
 *   M      rows, >= 0 (M == 0 returns MBN_OK, pointers may then be NULL);
 *          at most 2^31 - 1
 *   N      row width, 1 <= N <= MBN_RMSNORM_MAX_N
 *   eps    finite, >= 0 (added inside the square root)
 *   stream hipStream_t or NULL
 * x, w and y must be 2-byte aligned (an odd address is MBN_EUNSUPPORTED).
 * Launch path (same results to the documented tolerance, not bit-identical):
 * when N % 8 == 0 and every pointer is 16-byte aligned, the staged-row
 * kernels (16-byte row chunks); otherwise the any-width kernels. Those never
 * write outside the rows. When x and y sit at the same address modulo 16 and
 * either N >= 1024 (unless N % 4 == 0 with every pointer 8-byte aligned) or
 * N >= 256 with a pointer that is not 8-byte aligned, they copy the 16-byte
 * blocks that hold row elements (so they may read up to 14 bytes before and
 * after a row, inside those blocks, never another page); otherwise they access
 * groups of 4, 2 or 1 elements and read nothing outside the rows. The same
 * holds for add_rmsnorm_fwd (x, r, h and y at one address modulo 16),
 * layernorm_fwd and l2norm_fwd.
 * IEEE behaviour: a NaN in a row makes the row NaN; an infinite element makes
 * the finite elements of its row 0 and itself NaN; a zero row gives 0 when
 * eps > 0 and NaN when eps == 0. Rows whose sum of squares overflows fp32
 * (|x| above about 1.8e19) behave like rows holding an infinity.
 */
MBN_API int rmsnorm_fwd(const void* x, const void* w, void* y, int64_t M, int64_t N,
                        float eps, void* stream);

/*
 * add_rmsnorm_fwd -- residual add fused with RMSNorm (bf16).
 *
 * The residual add + norm fusion of "TorchInductor: from ATen IR to Triton
 * kernel", sections 14.25 and 14.27, on the staged-row kernel of
 * "[Inductor] Codegen Gluon", section 3.1. The residual stream is bf16, so
 * the sum is rounded and the norm is taken of what is stored:
 *     h[i,j] = bf16( x[i,j] + r[i,j] )
 *     y[i,j] = bf16( h[i,j] / sqrt( (1/N) sum_j h[i,j]^2 + eps ) * w[j] )
 *
 *   x, r   device, bf16 [M, N], read only (unless aliased by h or y)
 *   w      device, bf16 [N]
 *   h      device, bf16 [M, N], written (the updated residual stream)
 *   y      device, bf16 [M, N], written
 *   M, N, eps, stream: as for rmsnorm_fwd.
 * h and y may each coincide exactly with x or with r (in place); h and y must
 * not overlap each other, and no other overlap is allowed (MBN_EINVAL). All
 * five pointers must be 2-byte aligned (16-byte aligned with N % 8 == 0 for
 * the staged-row kernels).
 */
MBN_API int add_rmsnorm_fwd(const void* x, const void* r, const void* w, void* h, void* y,
                            int64_t M, int64_t N, float eps, void* stream);

/*
 * layernorm_fwd -- row-wise LayerNorm forward (bf16).
 *
 * The decomposition of "TorchInductor: from ATen IR to Triton kernel",
 * section 14.12.2 (var_mean, add eps, rsqrt, subtract, multiply, weight,
 * bias), and the LayerNorm entry of "[Inductor] Codegen Gluon", section 3.2
 * (the input is reused by the mean / variance reduction and by the affine
 * pass). Biased variance:
 *     mu  = (1/N) sum_j x[i,j],  var = (1/N) sum_j (x[i,j] - mu)^2
 *     y[i,j] = bf16( (x[i,j] - mu) / sqrt(var + eps) * w[j] + b[j] )
 * Both moments are taken from the LDS-staged row in fp32 (two passes).
 *
 *   x      device, bf16 [M, N];  w, b  device, bf16 [N];  y  device, bf16 [M, N]
 *   M, N, eps, stream: as for rmsnorm_fwd. y == x allowed; w and b must not
 *   overlap y. Pointer alignment and launch path as for rmsnorm_fwd.
 */
MBN_API int layernorm_fwd(const void* x, const void* w, const void* b, void* y, int64_t M,
                          int64_t N, float eps, void* stream);

/*
 * l2norm_fwd -- row-wise L2 normalization (bf16).
 *
 * The L2Norm entry of "[Inductor] Codegen Gluon", section 3.2 (one reduction,
 * then a scale by the inverse norm), with the usual eps guard:
 *     y[i,j] = bf16( x[i,j] / max( sqrt( sum_j x[i,j]^2 ), eps ) )
 * A NaN anywhere in a row makes the row NaN; eps = 0 and a zero row give NaN.
 *
 *   x, y   device, bf16 [M, N] (y == x allowed)
 *   M, N, eps, stream, pointer alignment, launch path: as for rmsnorm_fwd.
 */
MBN_API int l2norm_fwd(const void* x, void* y, int64_t M, int64_t N, float eps, void* stream);

/*
 * qk_norm_rope_fwd -- fused per-head RMSNorm + rotary embedding on the q and
 * k heads of a packed QKV tensor, in place.
 *
 * Defined by "[pretuned] Optimize fused_qk_norm_rope on B200", Summary (full
 * rotary case: the two rotary halves of each head are loaded once, the RMS is
 * taken over the whole head, the Q/K weight and the rotary embedding are
 * applied without a round trip through memory, and each half is stored once).
 * For token t, with D = head_dim and each q head (weight q_w) or k head
 * (weight k_w) holding x[0..D):
 *     rstd  = 1 / sqrt( mean_d x[d]^2 + eps ),   u[d] = x[d] * rstd * w[d]
 *     phi_i = positions[t] * theta^(-2i/D)        for i in [0, D/2)
 *     out[i]       = u[i]       * cos(phi_i) - u[i+D/2] * sin(phi_i)
 *     out[i+D/2]   = u[i+D/2]   * cos(phi_i) + u[i]     * sin(phi_i)
 * (rotate-half pairing, as in NeoX-style rotary embeddings). The angles, their
 * sine / cosine and the rotation's products are computed in fp64, the head's
 * sum of squares and rstd in fp32, with one rounding to bf16 at the store.
 *
 *   qkv        device, bf16 [T, (n_q_heads + 2*n_kv_heads) * head_dim], read
 *              and written in place. Per token: n_q_heads q heads, then
 *              n_kv_heads k heads, then n_kv_heads v heads; v is never read
 *              or written.
 *   q_w, k_w   device, bf16 [head_dim] each, shared by all q (k) heads
 *   positions  device, int64 [T]. Any value is accepted; it is converted to
 *              fp64 (exact for |position| <= 2^53). Parity with the fp64
 *              reference above (one bf16 ulp plus 1e-6) is established for
 *              |position| <= 1.23e8, i.e. angles up to ~1.2e8 rad. Beyond
 *              that the fp64 angle is itself uncertain by half an ulp of phi
 *              (7e-9 rad at 1e8 rad, 6e-8 rad near 1e9) on both sides, so the
 *              1e-6 absolute floor can no longer judge near-cancelling
 *              outputs; angles with |phi| >= 2^40 take the device library's
 *              sine and cosine.
 *   T          tokens, >= 0 (T == 0 returns MBN_OK); at most 2^31 - 1
 *   n_q_heads, n_kv_heads  >= 0
 *   head_dim   must equal MBN_QK_HEAD_DIM (odd values are MBN_EINVAL)
 *   eps        finite, >= 0;  theta  finite, > 0
 *   stream     hipStream_t or NULL
 * qkv, q_w and k_w must be 16-byte aligned, positions 8-byte aligned; q_w,
 * k_w and positions must not overlap the q/k part of qkv.
 */
MBN_API int qk_norm_rope_fwd(void* qkv, const void* q_w, const void* k_w,
                             const int64_t* positions, int64_t T, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, float eps, float theta,
                             void* stream);

/*
 * qk_norm_rope_partial_fwd -- qk_norm_rope_fwd with a rotary part shorter than
 * the head.
 *
 * "[pretuned] Optimize fused_qk_norm_rope on B200", Summary: with a partial
 * rotary dimension the full-head normalization is kept, since the values past
 * the rotary part must still be normalized. With R = rotary_dim:
 *     rstd and u[d] = x[d] * rstd * w[d] over the whole head (d < D)
 *     phi_i = positions[t] * theta^(-2i/R)        for i in [0, R/2)
 *     out[i]     = u[i]     * cos(phi_i) - u[i+R/2] * sin(phi_i)
 *     out[i+R/2] = u[i+R/2] * cos(phi_i) + u[i]     * sin(phi_i)
 *     out[d]     = u[d]                            for d in [R, D)
 * rotary_dim == head_dim is exactly qk_norm_rope_fwd.
 *
 *   rotary_dim  even, 0 < rotary_dim <= head_dim (else MBN_EINVAL); the
 *               kernels handle multiples of 16 (else MBN_EUNSUPPORTED)
 *   every other argument as for qk_norm_rope_fwd.
 */
MBN_API int qk_norm_rope_partial_fwd(void* qkv, const void* q_w, const void* k_w,
                                     const int64_t* positions, int64_t T, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t rotary_dim,
                                     float eps, float theta, void* stream);

/*
 * fp16 variants -- the same operators on IEEE binary16 data.
 *
 * "[Inductor] Codegen Gluon", section 3.2, lists fp16 inputs among the
 * broadened cases of the reused-input norms. Every tensor argument that is
 * bf16 above is binary16 here (x, r, w, b, h, y, qkv, q_w, k_w); the formulas,
 * layouts, alias rules, validation and status codes are those of the bf16
 * entry point of the same name; arithmetic is fp32 (fp64 for the angles and
 * rotation products) and each output is rounded once to nearest even in
 * binary16 (overflow gives +-inf). The full-rotary QK case is
 * qk_norm_rope_partial_fwd_f16 with rotary_dim == head_dim.
 */
MBN_API int rmsnorm_fwd_f16(const void* x, const void* w, void* y, int64_t M, int64_t N,
                            float eps, void* stream);
MBN_API int add_rmsnorm_fwd_f16(const void* x, const void* r, const void* w, void* h, void* y,
                                int64_t M, int64_t N, float eps, void* stream);
MBN_API int layernorm_fwd_f16(const void* x, const void* w, const void* b, void* y, int64_t M,
                              int64_t N, float eps, void* stream);
MBN_API int l2norm_fwd_f16(const void* x, void* y, int64_t M, int64_t N, float eps,
                           void* stream);
MBN_API int qk_norm_rope_partial_fwd_f16(void* qkv, const void* q_w, const void* k_w,
                                         const int64_t* positions, int64_t T, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t rotary_dim,
                                         float eps, float theta, void* stream);

/*
 * Timed variants -- rmsnorm_fwd and qk_norm_rope_fwd with kernel-execution
 * timestamps.
 *
 * The operation, arguments, validation and status codes are exactly those of
 * the entry point without the suffix. In addition, the call's first kernel
 * records start_event when it starts executing on the GPU and its last kernel
 * records stop_event when it has finished (hipExtLaunchKernel), so that
 * hipEventElapsedTime(start_event, stop_event) is the duration of the call's
 * own kernels: what a bandwidth figure of the operation divides its bytes by,
 * the same interval a kernel trace reports. A hipEventRecord before and after
 * the plain call measures more: the queue packets of the two records and the
 * kernel's dispatch after the first.
 *
 *   start_event, stop_event  hipEvent_t (as void*), created by the caller on
 *              the stream's device, both non-NULL (else MBN_EINVAL). They are
 *              left unrecorded when the call launches nothing (an empty input)
 *              or returns an error.
 * Meant for eager timing: the events are attached to the dispatches, which a
 * HIP graph capture need not support; capture the plain entry points.
 */
MBN_API int rmsnorm_fwd_timed(const void* x, const void* w, void* y, int64_t M, int64_t N,
                              float eps, void* stream, void* start_event, void* stop_event);
MBN_API int qk_norm_rope_fwd_timed(void* qkv, const void* q_w, const void* k_w,
                                   const int64_t* positions, int64_t T, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, float eps, float theta,
                                   void* stream, void* start_event, void* stop_event);

/* Static, NUL-terminated description of a status code (never NULL). */
MBN_API const char* mbn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MBN_H */
