// Read-stream probe for gfx950: the rate at which one launch can read a
// buffer from HBM when it does nothing else. The benchmark times it on the
// same bytes as a verification call to give that call a measured ceiling.
// It is measurement tooling, not part of the verifier.
//
// A workgroup (4 waves) owns a run of 4 KiB chunks; each wave reads chunks
// c, c + 4, ... with four 16-byte loads per lane, the next chunk's loads
// issued before the current one is folded in. The fold is an xor, so no
// load is dead; one word per workgroup is written.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 4096;
constexpr int kLoads = kChunk / (64 * 16);

__device__ __forceinline__ void issue(const uint4* base, size_t ch, uint4 (&r)[kLoads]) {
#pragma unroll
  for (int j = 0; j < kLoads; ++j) r[j] = base[ch * (kChunk / 16) + j * 64];
}

__device__ __forceinline__ uint32_t fold(const uint4 (&r)[kLoads]) {
  uint32_t v = 0u;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) v ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
  return v;
}

// Two alternating buffers: the loads of the next chunk are issued before
// the current one is folded (past the run's end the current chunk is
// issued again, so every iteration has the same loads in flight).
__global__ __launch_bounds__(kThreads) void probe_kernel(const uint4* __restrict__ p, size_t n_chunk,
                                                         int cpw, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t c_lo = (size_t)blockIdx.x * cpw;
  const size_t c_hi = c_lo + cpw < n_chunk ? c_lo + cpw : n_chunk;
  const uint4* base = p + lane;
  uint32_t acc = 0u;
  size_t ch = c_lo + wave;
  if (ch < c_hi) {
    uint4 a[kLoads], b[kLoads];
    issue(base, ch, a);
    while (true) {
      size_t nx = ch + kWaves;
      bool more = nx < c_hi;
      issue(base, more ? nx : ch, b);
      acc ^= fold(a);
      ch = nx;
      if (!more) break;
      nx = ch + kWaves;
      more = nx < c_hi;
      issue(base, more ? nx : ch, a);
      acc ^= fold(b);
      ch = nx;
      if (!more) break;
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  __shared__ uint32_t s[kWaves];
  if (lane == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 4096, 16-byte aligned device memory) once on
// stream; out receives one word per workgroup (at least
// sv_probe_workgroups(bytes) words). Returns 0, or -1 for bad arguments, -2
// when the launch fails.
int sv_probe_workgroups(size_t bytes) {
  const size_t n_chunk = bytes / kChunk;
  const size_t cpw = (n_chunk + 8191) / 8192 > (size_t)kWaves ? (n_chunk + 8191) / 8192 : kWaves;
  return (int)((n_chunk + cpw - 1) / cpw);
}

int sv_probe_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out || bytes == 0 || bytes % kChunk != 0 || (uintptr_t)buf % 16 != 0) return -1;
  const size_t n_chunk = bytes / kChunk;
  const size_t cpw = (n_chunk + 8191) / 8192 > (size_t)kWaves ? (n_chunk + 8191) / 8192 : kWaves;
  const unsigned grid = (unsigned)((n_chunk + cpw - 1) / cpw);
  hipLaunchKernelGGL(probe_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), n_chunk, (int)cpw, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
