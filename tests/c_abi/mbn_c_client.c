/*
 * A plain C client of libmbn.so: device memory from the HIP runtime,
 * operators through the C entry points of mbn.h, no PyTorch. The GPU tests
 * load it (built into tests/c_abi/libmbn_c_client.so) and compare what it
 * returns with the fp64 oracle.
 *
 * Each function copies host arrays to the device, runs one operator on the
 * null stream, copies the result back and frees what it allocated. Returns
 * the operator's mbn status, or 100 + the failing HIP error code.
 */
#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "mbn.h"

#define HIP_OK(call)                          \
  do {                                        \
    hipError_t e_ = (call);                   \
    if (e_ != hipSuccess) {                   \
      status = 100 + (int)e_;                 \
      goto done;                              \
    }                                         \
  } while (0)

/* y[M, N] = RMSNorm(x[M, N]) * w[N]; 16-bit arrays as raw bits. */
int mbn_c_client_rmsnorm(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t M, int64_t N,
                         float eps) {
  int status = 0;
  void *dx = NULL, *dw = NULL, *dy = NULL;
  const size_t bytes = (size_t)M * (size_t)N * 2;
  HIP_OK(hipMalloc(&dx, bytes));
  HIP_OK(hipMalloc(&dw, (size_t)N * 2));
  HIP_OK(hipMalloc(&dy, bytes));
  HIP_OK(hipMemcpy(dx, x, bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, w, (size_t)N * 2, hipMemcpyHostToDevice));
  status = rmsnorm_fwd(dx, dw, dy, M, N, eps, NULL);
  if (status != MBN_OK) goto done;
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(y, dy, bytes, hipMemcpyDeviceToHost));
done:
  hipFree(dx);
  hipFree(dw);
  hipFree(dy);
  return status;
}

/* qkv[T, (Hq + 2 Hkv) * 128] modified in place (q and k heads). */
int mbn_c_client_qk_norm_rope(uint16_t* qkv, const uint16_t* q_w, const uint16_t* k_w,
                              const int64_t* positions, int64_t T, int32_t n_q_heads,
                              int32_t n_kv_heads, float eps, float theta) {
  int status = 0;
  void *dq = NULL, *dqw = NULL, *dkw = NULL, *dpos = NULL;
  const size_t bytes = (size_t)T * (size_t)(n_q_heads + 2 * n_kv_heads) * MBN_QK_HEAD_DIM * 2;
  HIP_OK(hipMalloc(&dq, bytes));
  HIP_OK(hipMalloc(&dqw, MBN_QK_HEAD_DIM * 2));
  HIP_OK(hipMalloc(&dkw, MBN_QK_HEAD_DIM * 2));
  HIP_OK(hipMalloc(&dpos, (size_t)T * 8));
  HIP_OK(hipMemcpy(dq, qkv, bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dqw, q_w, MBN_QK_HEAD_DIM * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkw, k_w, MBN_QK_HEAD_DIM * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dpos, positions, (size_t)T * 8, hipMemcpyHostToDevice));
  status = qk_norm_rope_fwd(dq, dqw, dkw, (const int64_t*)dpos, T, n_q_heads, n_kv_heads, MBN_QK_HEAD_DIM,
                            eps, theta, NULL);
  if (status != MBN_OK) goto done;
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(qkv, dq, bytes, hipMemcpyDeviceToHost));
done:
  hipFree(dq);
  hipFree(dqw);
  hipFree(dkw);
  hipFree(dpos);
  return status;
}

/* The status of a call the library must reject on the host (null x). */
int mbn_c_client_reject(void) { return rmsnorm_fwd(NULL, NULL, NULL, 4, 8, 1e-6f, NULL); }
