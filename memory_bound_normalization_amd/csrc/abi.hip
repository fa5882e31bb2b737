// C entry points of libmbn.so: argument validation (host only, before any HIP
// call) and dispatch to the kernel launchers. The contract of every function
// is documented in include/mbn.h.
#include <math.h>
#include <stdint.h>

#include "../../include/mbn.h"
#include "kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

bool valid_eps(float eps) { return isfinite(eps) && eps >= 0.0f; }

// Checks shared by the row norms: sizes, eps, and the widths and row counts
// the kernels handle. Returns MBN_OK when a launch should follow, -1 for an
// empty input (nothing to do), or a status.
int check_rows(int64_t M, int64_t N, float eps) {
  if (M < 0 || N <= 0 || !valid_eps(eps)) return MBN_EINVAL;
  if (M == 0) return -1;
  if (N > MBN_RMSNORM_MAX_N || M > 0x7fffffffLL) return MBN_EUNSUPPORTED;
  return MBN_OK;
}

// An output may coincide exactly with an input of the same shape (in place);
// any other overlap is invalid.
bool bad_alias(const void* out, const void* in, int64_t bytes) {
  return out != in && overlap(out, bytes, in, bytes);
}

// Row-norm pointers must be element (2-byte) aligned; null ones (unused
// operands) pass.
bool elem_aligned(const void* p) { return aligned(p, 2); }
bool chunk_aligned(const void* p) { return aligned(p, 16); }

// Launch a row norm: the staged-row kernels when every row is whole 16-byte
// chunks (N % 8 == 0, all pointers 16-byte aligned), else the any-width
// kernels. Unused operands are null.
int launch(mbn::Norm mode, mbn::Storage dt, const void* x, const void* r, const void* w,
           const void* b, void* h, void* y, int64_t M, int64_t N, float eps, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool chunked = N % 8 == 0 && chunk_aligned(x) && chunk_aligned(r) && chunk_aligned(w) &&
                       chunk_aligned(b) && chunk_aligned(h) && chunk_aligned(y);
  hipError_t err;
  if (chunked) {
    mbn::RowNormArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.r = static_cast<const uint16_t*>(r);
    a.w = static_cast<const uint16_t*>(w);
    a.b = static_cast<const uint16_t*>(b);
    a.h = static_cast<uint16_t*>(h);
    a.y = static_cast<uint16_t*>(y);
    a.M = M;
    a.nchunk = (int)(N / 8);
    a.eps = eps;
    err = mbn::launch_rownorm(mode, dt, a, s);
  } else {
    mbn::RowNormAnyArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.r = static_cast<const uint16_t*>(r);
    a.w = static_cast<const uint16_t*>(w);
    a.b = static_cast<const uint16_t*>(b);
    a.h = static_cast<uint16_t*>(h);
    a.y = static_cast<uint16_t*>(y);
    a.M = M;
    a.n = (int)N;
    a.eps = eps;
    err = mbn::launch_rownorm_any(mode, dt, a, s);
  }
  return err == hipSuccess ? MBN_OK : MBN_EHIP;
}

// Entry-point bodies, shared by the bf16 and fp16 variants (the storage type
// changes nothing in the checks: both are 2 bytes per element).
int rmsnorm_impl(mbn::Storage dt, const void* x, const void* w, void* y, int64_t M, int64_t N,
                 float eps, void* stream) {
  const int st = check_rows(M, N, eps);
  if (st != MBN_OK) return st < 0 ? MBN_OK : st;
  if (!x || !w || !y) return MBN_EINVAL;
  if (!elem_aligned(x) || !elem_aligned(w) || !elem_aligned(y)) return MBN_EUNSUPPORTED;
  const int64_t bytes = M * N * 2;
  if (bad_alias(y, x, bytes) || overlap(w, N * 2, y, bytes)) return MBN_EINVAL;
  return launch(mbn::Norm::kRms, dt, x, nullptr, w, nullptr, nullptr, y, M, N, eps, stream);
}

int add_rmsnorm_impl(mbn::Storage dt, const void* x, const void* r, const void* w, void* h,
                     void* y, int64_t M, int64_t N, float eps, void* stream) {
  const int st = check_rows(M, N, eps);
  if (st != MBN_OK) return st < 0 ? MBN_OK : st;
  if (!x || !r || !w || !h || !y) return MBN_EINVAL;
  if (!elem_aligned(x) || !elem_aligned(r) || !elem_aligned(w) || !elem_aligned(h) ||
      !elem_aligned(y))
    return MBN_EUNSUPPORTED;
  const int64_t bytes = M * N * 2;
  if (overlap(h, bytes, y, bytes) || bad_alias(h, x, bytes) || bad_alias(h, r, bytes) ||
      bad_alias(y, x, bytes) || bad_alias(y, r, bytes) || overlap(w, N * 2, h, bytes) ||
      overlap(w, N * 2, y, bytes))
    return MBN_EINVAL;
  return launch(mbn::Norm::kAddRms, dt, x, r, w, nullptr, h, y, M, N, eps, stream);
}

int layernorm_impl(mbn::Storage dt, const void* x, const void* w, const void* b, void* y,
                   int64_t M, int64_t N, float eps, void* stream) {
  const int st = check_rows(M, N, eps);
  if (st != MBN_OK) return st < 0 ? MBN_OK : st;
  if (!x || !w || !b || !y) return MBN_EINVAL;
  if (!elem_aligned(x) || !elem_aligned(w) || !elem_aligned(b) || !elem_aligned(y))
    return MBN_EUNSUPPORTED;
  const int64_t bytes = M * N * 2;
  if (bad_alias(y, x, bytes) || overlap(w, N * 2, y, bytes) || overlap(b, N * 2, y, bytes))
    return MBN_EINVAL;
  return launch(mbn::Norm::kLayer, dt, x, nullptr, w, b, nullptr, y, M, N, eps, stream);
}

int l2norm_impl(mbn::Storage dt, const void* x, void* y, int64_t M, int64_t N, float eps,
                void* stream) {
  const int st = check_rows(M, N, eps);
  if (st != MBN_OK) return st < 0 ? MBN_OK : st;
  if (!x || !y) return MBN_EINVAL;
  if (!elem_aligned(x) || !elem_aligned(y)) return MBN_EUNSUPPORTED;
  if (bad_alias(y, x, M * N * 2)) return MBN_EINVAL;
  return launch(mbn::Norm::kL2, dt, x, nullptr, nullptr, nullptr, nullptr, y, M, N, eps, stream);
}

int qk_impl(mbn::Storage dt, void* qkv, const void* q_w, const void* k_w,
            const int64_t* positions, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
            int32_t head_dim, int32_t rotary_dim, float eps, float theta, void* stream) {
  if (T < 0 || n_q_heads < 0 || n_kv_heads < 0 || head_dim <= 0 || (head_dim & 1))
    return MBN_EINVAL;
  if (rotary_dim <= 0 || (rotary_dim & 1) || rotary_dim > head_dim) return MBN_EINVAL;
  if (!valid_eps(eps) || !isfinite(theta) || !(theta > 0.0f)) return MBN_EINVAL;
  if (head_dim != MBN_QK_HEAD_DIM || rotary_dim % 16 != 0) return MBN_EUNSUPPORTED;
  const int64_t heads = (int64_t)n_q_heads + n_kv_heads;
  if (T == 0 || heads == 0) return MBN_OK;
  if (!qkv || !positions || (n_q_heads > 0 && !q_w) || (n_kv_heads > 0 && !k_w))
    return MBN_EINVAL;
  if (T > 0x7fffffffLL || heads > (1 << 20)) return MBN_EUNSUPPORTED;
  if (!aligned(qkv, 16) || (q_w && !aligned(q_w, 16)) || (k_w && !aligned(k_w, 16)) ||
      !aligned(positions, 8))
    return MBN_EUNSUPPORTED;
  // The q/k part of the last token ends before its v heads; any read-only input
  // inside the span [qkv, end of the last token's k heads) is rejected.
  const int64_t row_bytes = ((int64_t)n_q_heads + 2 * (int64_t)n_kv_heads) * head_dim * 2;
  const int64_t span = (T - 1) * row_bytes + heads * head_dim * 2;
  const int64_t wbytes = (int64_t)head_dim * 2;
  if ((n_q_heads > 0 && overlap(q_w, wbytes, qkv, span)) ||
      (n_kv_heads > 0 && overlap(k_w, wbytes, qkv, span)) || overlap(positions, T * 8, qkv, span))
    return MBN_EINVAL;
  const hipError_t err =
      mbn::launch_qk_norm_rope(dt, qkv, q_w, k_w, positions, T, n_q_heads, n_kv_heads,
                               rotary_dim, eps, theta, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MBN_OK : MBN_EHIP;
}

constexpr mbn::Storage kBf16 = mbn::Storage::kBf16;
constexpr mbn::Storage kF16 = mbn::Storage::kF16;

// Points the calling thread's timing slot at a call's events for the duration
// of that call (the *_timed entry points).
class TimedCall {
 public:
  TimedCall(void* start, void* stop)
      : t_{static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)},
        prev_(mbn::launch_timing()) {
    mbn::launch_timing() = &t_;
  }
  ~TimedCall() { mbn::launch_timing() = prev_; }
  TimedCall(const TimedCall&) = delete;
  TimedCall& operator=(const TimedCall&) = delete;

 private:
  mbn::LaunchTiming t_;
  mbn::LaunchTiming* prev_;
};

}  // namespace

extern "C" {

MBN_API int rmsnorm_fwd(const void* x, const void* w, void* y, int64_t M, int64_t N, float eps,
                        void* stream) {
  return rmsnorm_impl(kBf16, x, w, y, M, N, eps, stream);
}

MBN_API int add_rmsnorm_fwd(const void* x, const void* r, const void* w, void* h, void* y,
                            int64_t M, int64_t N, float eps, void* stream) {
  return add_rmsnorm_impl(kBf16, x, r, w, h, y, M, N, eps, stream);
}

MBN_API int layernorm_fwd(const void* x, const void* w, const void* b, void* y, int64_t M,
                          int64_t N, float eps, void* stream) {
  return layernorm_impl(kBf16, x, w, b, y, M, N, eps, stream);
}

MBN_API int l2norm_fwd(const void* x, void* y, int64_t M, int64_t N, float eps, void* stream) {
  return l2norm_impl(kBf16, x, y, M, N, eps, stream);
}

MBN_API int qk_norm_rope_partial_fwd(void* qkv, const void* q_w, const void* k_w,
                                     const int64_t* positions, int64_t T, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t rotary_dim,
                                     float eps, float theta, void* stream) {
  return qk_impl(kBf16, qkv, q_w, k_w, positions, T, n_q_heads, n_kv_heads, head_dim, rotary_dim,
                 eps, theta, stream);
}

MBN_API int qk_norm_rope_fwd(void* qkv, const void* q_w, const void* k_w,
                             const int64_t* positions, int64_t T, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim, float eps, float theta,
                             void* stream) {
  return qk_impl(kBf16, qkv, q_w, k_w, positions, T, n_q_heads, n_kv_heads, head_dim, head_dim,
                 eps, theta, stream);
}

MBN_API int rmsnorm_fwd_f16(const void* x, const void* w, void* y, int64_t M, int64_t N,
                            float eps, void* stream) {
  return rmsnorm_impl(kF16, x, w, y, M, N, eps, stream);
}

MBN_API int add_rmsnorm_fwd_f16(const void* x, const void* r, const void* w, void* h, void* y,
                                int64_t M, int64_t N, float eps, void* stream) {
  return add_rmsnorm_impl(kF16, x, r, w, h, y, M, N, eps, stream);
}

MBN_API int layernorm_fwd_f16(const void* x, const void* w, const void* b, void* y, int64_t M,
                              int64_t N, float eps, void* stream) {
  return layernorm_impl(kF16, x, w, b, y, M, N, eps, stream);
}

MBN_API int l2norm_fwd_f16(const void* x, void* y, int64_t M, int64_t N, float eps,
                           void* stream) {
  return l2norm_impl(kF16, x, y, M, N, eps, stream);
}

MBN_API int qk_norm_rope_partial_fwd_f16(void* qkv, const void* q_w, const void* k_w,
                                         const int64_t* positions, int64_t T, int32_t n_q_heads,
                                         int32_t n_kv_heads, int32_t head_dim, int32_t rotary_dim,
                                         float eps, float theta, void* stream) {
  return qk_impl(kF16, qkv, q_w, k_w, positions, T, n_q_heads, n_kv_heads, head_dim, rotary_dim,
                 eps, theta, stream);
}

MBN_API int rmsnorm_fwd_timed(const void* x, const void* w, void* y, int64_t M, int64_t N,
                              float eps, void* stream, void* start_event, void* stop_event) {
  if (!start_event || !stop_event) return MBN_EINVAL;
  TimedCall timed(start_event, stop_event);
  return rmsnorm_impl(kBf16, x, w, y, M, N, eps, stream);
}

MBN_API int qk_norm_rope_fwd_timed(void* qkv, const void* q_w, const void* k_w,
                                   const int64_t* positions, int64_t T, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, float eps, float theta,
                                   void* stream, void* start_event, void* stop_event) {
  if (!start_event || !stop_event) return MBN_EINVAL;
  TimedCall timed(start_event, stop_event);
  return qk_impl(kBf16, qkv, q_w, k_w, positions, T, n_q_heads, n_kv_heads, head_dim, head_dim,
                 eps, theta, stream);
}

MBN_API const char* mbn_strerror(int status) {
  switch (status) {
    case MBN_OK: return "success";
    case MBN_EINVAL: return "invalid argument";
    case MBN_EUNSUPPORTED: return "unsupported shape, alignment or head size";
    case MBN_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
