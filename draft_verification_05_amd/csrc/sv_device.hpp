// Device building blocks for the gfx950 verifier: Philox, 128-bit logits
// loads with bf16 widening, wave64 / workgroup reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;              // one workgroup = 4 wave64s
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_inff();

// ------------------------------------------------------------- Philox ---
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): per round the 128-bit
// products of words 0 and 2 with the two multipliers are mixed with words
// 1 and 3 and the round key; the key advances by the Weyl increments.
struct Philox4 { uint64_t w0, w1, w2, w3; };

__device__ inline Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                        uint64_t k0, uint64_t k1) {
  const uint64_t kMul0 = 0xD2E7470EE14C6C93ull, kMul1 = 0xCA5A826395121157ull;
  const uint64_t kInc0 = 0x9E3779B97F4A7C15ull, kInc1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += kInc0; k1 += kInc1; }
    const uint64_t hi0 = __umul64hi(kMul0, c0), lo0 = kMul0 * c0;
    const uint64_t hi1 = __umul64hi(kMul1, c2), lo1 = kMul1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return {c0, c1, c2, c3};
}

// Top 24 bits as a float in [0, 1): exact in fp32.
__device__ inline float top24(uint64_t w) { return (float)(uint32_t)(w >> 40) * 0x1p-24f; }

// ------------------------------------------------------------- loads ---
enum { kF32 = 0, kBF16 = 1 };

template <int DT> struct Elem;
template <> struct Elem<kF32>  { static constexpr int kPerVec = 4; static constexpr int kBytes = 4; };
template <> struct Elem<kBF16> { static constexpr int kPerVec = 8; static constexpr int kBytes = 2; };

// bf16 is the upper half of an fp32: widening is a shift or a mask.
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ inline void load_vec16(const char* p, float* out);

template <>
__device__ inline void load_vec16<kF32>(const char* p, float* out) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

template <>
__device__ inline void load_vec16<kBF16>(const char* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
  out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
  out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
  out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
}

template <int DT>
__device__ inline float load_one(const char* row, int64_t e) {
  if constexpr (DT == kF32) {
    return reinterpret_cast<const float*>(row)[e];
  } else {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[e] << 16);
  }
}

// A segment is kThreads * U vectors of Elem::kPerVec logits. Thread t holds
// vectors t, t + kThreads, ..., so each of the U loads of a wave is one
// contiguous 1 KiB run. Elements at or past V read as -inf.
template <int DT, int U, bool kVec>
__device__ inline void load_segment(const char* row, int64_t seg0, int V,
                                    float (&x)[U * Elem<DT>::kPerVec]) {
  constexpr int kPer = Elem<DT>::kPerVec;
  constexpr int kLen = kThreads * U * kPer;
  const int tid = threadIdx.x;
  if (kVec && seg0 + kLen <= V) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t e0 = seg0 + (int64_t)(j * kThreads + tid) * kPer;
      load_vec16<DT>(row + e0 * Elem<DT>::kBytes, &x[j * kPer]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t e0 = seg0 + (int64_t)(j * kThreads + tid) * kPer;
      if (kVec && e0 + kPer <= V) {
        load_vec16<DT>(row + e0 * Elem<DT>::kBytes, &x[j * kPer]);
      } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k)
          x[j * kPer + k] = (e0 + k < V) ? load_one<DT>(row, e0 + k) : kNegInf;
      }
    }
  }
}

// ------------------------------------------------------ reductions ---
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two (max, sum of 2^(y - max)) pairs.
__device__ inline void ms_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) { m = mn; s = 0.f; return; }
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

__device__ inline void wave_reduce_ms(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const float s2 = __shfl_xor(s, o);
    ms_merge(m, s, m2, s2);
  }
}

// (value, index): larger value wins, lower index on ties.
__device__ inline void am_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ inline void wave_reduce_am(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o);
    const int i2 = __shfl_xor(i, o);
    am_merge(v, i, v2, i2);
  }
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Workgroup inclusive scan; `total` is the same value in every thread.
// `lds` holds kWaves floats. Ends with a barrier so `lds` can be reused.
__device__ inline float block_incl_scan(float v, float* lds, float& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float incl = wave_incl_scan(v);
  if (lane == 63) lds[w] = incl;
  __syncthreads();
  float off = 0.f, tot = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const float t = lds[i];
    if (i < w) off += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return incl + off;
}

// Workgroup sum, identical in every thread; ends with a barrier.
__device__ inline float block_sum(float v, float* lds) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) tot += lds[i];
  __syncthreads();
  return tot;
}

}  // namespace sv
