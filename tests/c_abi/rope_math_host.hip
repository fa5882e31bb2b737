// Host build of the rotary-angle functions of the fused QK-norm + RoPE kernel
// (memory_bound_normalization_amd/csrc/rope_math.h): the code the kernel runs,
// called on the CPU so the tests can hold it against high-precision values.
#include <stdint.h>

#include "../../memory_bound_normalization_amd/csrc/rope_math.h"

extern "C" {

// s[i], c[i] = sin, cos of phi[i] for i < n (sincos_reduced).
__attribute__((visibility("default"))) void mbn_test_sincos(const double* phi, double* s, double* c, int64_t n) {
  for (int64_t i = 0; i < n; ++i) mbn::sincos_reduced(phi[i], s + i, c + i);
}

// out[i] = theta^(-2i/R) for i < R/2, as the launcher and the kernel form it.
__attribute__((visibility("default"))) void mbn_test_inv_freq(float theta, int rotary_dim, double* out) {
  const mbn::InvFreqPowers ip = mbn::rope_inv_freq_powers(theta, rotary_dim);
  for (int i = 0; i < rotary_dim / 2; ++i) out[i] = mbn::rope_inv_freq(ip, i);
}

}  // extern "C"
