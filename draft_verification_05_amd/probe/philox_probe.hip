// Test-only kernel: the library's device Philox4x64-10 (sv_device.hpp) on
// caller-given counters and keys, so a test can compare it word for word
// with an independent implementation. Not part of the verifier.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../csrc/sv_device.hpp"

namespace {

__global__ void philox_words_kernel(const uint64_t* ctr, const uint64_t* key, uint64_t* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const sv::Philox4 w = sv::philox4x64_10(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3],
                                          key[2 * i], key[2 * i + 1]);
  out[4 * i] = w.w0;
  out[4 * i + 1] = w.w1;
  out[4 * i + 2] = w.w2;
  out[4 * i + 3] = w.w3;
}

}  // namespace

// ctr [n, 4], key [n, 2], out [n, 4]: device uint64 arrays; n in [1, 2^31).
// Returns 0, -1 for a NULL pointer or n out of range, -7 for a failed launch.
extern "C" int sv_philox_words(const uint64_t* ctr, const uint64_t* key, uint64_t* out, int64_t n,
                               void* stream) {
  if (!ctr || !key || !out) return -1;
  if (n < 1 || n >= (int64_t)1 << 31) return -1;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(philox_words_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     ctr, key, out, n);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
