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

// A chunk is 4 KiB of consecutive logits (2048 bf16 or 1024 fp32): the
// unit of one partial, and what one wave reads per step (four 16-byte
// loads per lane, each load instruction one contiguous 1 KiB of the wave).
constexpr int kChunkBytes = 4096;
constexpr int kLoadsPerLane = kChunkBytes / (64 * 16);

template <int DT> struct Chunk {
  static constexpr int kPer = Elem<DT>::kPerVec;             // logits per 16-byte load
  static constexpr int kElems = kChunkBytes / Elem<DT>::kBytes;
  static constexpr int kPerLane = kElems / 64;                // logits per lane
  static constexpr int kPerThread = kElems / kThreads;        // when a workgroup reads it
};

// Raw 16-byte vectors of one chunk for one lane: vector j covers logits
// c0 + (j * 64 + lane) * kPer ... + kPer - 1.
struct ChunkRaw { uint4 v[kLoadsPerLane]; };

template <int DT>
__device__ __forceinline__ void issue_chunk(const char* row, int64_t c0, ChunkRaw& r) {
  constexpr int kPer = Elem<DT>::kPerVec;
  const char* p = row + (c0 + (int64_t)(threadIdx.x & 63) * kPer) * Elem<DT>::kBytes;
#pragma unroll
  for (int j = 0; j < kLoadsPerLane; ++j)
    r.v[j] = *reinterpret_cast<const uint4*>(p + j * 64 * 16);
}

// Grammar bitmask words of one chunk: vector j of the lane (logits
// c0 + (j * 64 + lane) * kPer ...) has its kPer bits in word
// (c0 + (j * 64 + lane) * kPer) / 32 (a chunk starts on a word, a vector
// never straddles one). Word indices past the row's last word are clamped
// (those logits read as -inf anyway).
struct MaskRaw { uint32_t w; };

// One coalesced load of a chunk's bitmask: lane l holds word l of it (a
// chunk starts on a word: 64 words for bf16, 32 for fp32, where lanes
// 32..63 repeat lanes 0..31). Word indices past the row's last word are
// clamped (those logits read as -inf anyway).
template <int DT>
__device__ __forceinline__ void issue_mask(const uint32_t* mrow, int64_t c0, int n_words, MaskRaw& m) {
  constexpr int kWords = Chunk<DT>::kElems / 32;
  const int64_t wi = (c0 >> 5) + ((threadIdx.x & 63) % kWords);
  m.w = mrow[wi < n_words ? wi : n_words - 1];
}

// Disallowed logits of a chunk become -inf in the packed words. The kPer
// bits of the lane's vector j sit in word (j * 64 + lane) * kPer / 32 of the
// chunk's mask, fetched from the lane that loaded it; after the shift bit k
// allows logit k of the vector. Per 32-bit word one bitfield insert against
// the -inf pattern. Every lane of the wave must be active.
template <int DT>
__device__ __forceinline__ void apply_mask(ChunkRaw& r, const MaskRaw& m) {
  constexpr int kPer = Elem<DT>::kPerVec;
  const int lane = threadIdx.x & 63;
  const uint32_t shift = (lane * kPer) & 31;
#pragma unroll
  for (int j = 0; j < kLoadsPerLane; ++j) {
    const int src = ((j * 64 + lane) * kPer) >> 5;   // < 64: a chunk's mask has at most 64 words
    const uint32_t bits = (uint32_t)__shfl((int)m.w, src) >> shift;
    auto blend = [bits](uint32_t& w, int q) {
      uint32_t keep;
      if constexpr (DT == kF32) {
        keep = 0u - ((bits >> q) & 1u);                               // 0 or all ones
      } else {
        keep = ((0u - ((bits >> (2 * q)) & 1u)) & 0x0000FFFFu) |
               ((0u - ((bits >> (2 * q + 1)) & 1u)) & 0xFFFF0000u);
      }
      const uint32_t inf = DT == kF32 ? 0xFF800000u : 0xFF80FF80u;
      w = (w & keep) | (inf & ~keep);
    };
    blend(r.v[j].x, 0);
    blend(r.v[j].y, 1);
    blend(r.v[j].z, 2);
    blend(r.v[j].w, 3);
  }
}

// Same layout as issue_chunk with bounds checks: a row's last, partial
// chunk (16-byte loads for the vectors inside the row when kVec) and rows
// that are not 16-byte aligned (element loads). Logits at or past V read as
// -inf (bf16 0xFF80, fp32 0xFF800000).
template <int DT, bool kVec>
__device__ __forceinline__ void load_chunk_checked(const char* row, int64_t c0, int V, ChunkRaw& r) {
  constexpr int kPer = Elem<DT>::kPerVec;
#pragma unroll
  for (int j = 0; j < kLoadsPerLane; ++j) {
    const int64_t e0 = c0 + (int64_t)(j * 64 + (threadIdx.x & 63)) * kPer;
    if (kVec && e0 + kPer <= V) {
      r.v[j] = *reinterpret_cast<const uint4*>(row + e0 * Elem<DT>::kBytes);
      continue;
    }
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (DT == kF32) {
        const int64_t e = e0 + q;
        w[q] = e < V ? __float_as_uint(load_one<DT>(row, e)) : 0xFF800000u;
      } else {
        const int64_t e = e0 + 2 * q;
        const uint32_t lo = e < V ? (uint32_t)reinterpret_cast<const uint16_t*>(row)[e] : 0xFF80u;
        const uint32_t hi = e + 1 < V ? (uint32_t)reinterpret_cast<const uint16_t*>(row)[e + 1] : 0xFF80u;
        w[q] = lo | (hi << 16);
      }
    }
    r.v[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// A whole workgroup reads one chunk: thread t holds logits
// c0 + t * kPerThread ... + kPerThread - 1, in index order.
template <int DT, bool kVec>
__device__ inline void load_chunk_wg(const char* row, int64_t c0, int V,
                                     float (&x)[Chunk<DT>::kPerThread]) {
  constexpr int kPT = Chunk<DT>::kPerThread;
  const int64_t e0 = c0 + (int64_t)threadIdx.x * kPT;
  if (kVec && e0 + kPT <= V) {
    load_vec16<DT>(row + e0 * Elem<DT>::kBytes, x);    // kPerThread logits = one 16-byte vector
  } else {
#pragma unroll
    for (int k = 0; k < kPT; ++k)
      x[k] = (e0 + k < V) ? load_one<DT>(row, e0 + k) : kNegInf;
  }
}

// ------------------------------------------------------ reductions ---
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave64 reductions on the DPP network: inside each row of 16 lanes, lane i
// meets lanes i^1, i^2 (quad permutes), then 7-i (half-row mirror) and 15-i
// (row mirror), after which every lane holds its row's result; the four
// row results are then combined through scalar reads. No LDS traffic.
template <int kCtrl>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
template <int kCtrl>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ inline float wave_max_all(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Sum over the wave, same value in every lane (fixed association order).
__device__ inline float wave_sum_all(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Inclusive prefix sum over the 64 lanes in lane order: Kogge-Stone row
// shifts by 1, 2, 4, 8 inside each row of 16, then row 15 broadcast into
// rows 1 and 3 and lane 31 into rows 2 and 3.
__device__ inline float wave_scan_incl(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}

// Lowest / highest lane whose predicate holds, -1 if none (wave-uniform).
__device__ inline int first_lane(bool p) {
  const unsigned long long m = __ballot(p);
  return m ? __builtin_ctzll(m) : -1;
}
__device__ inline int last_lane(bool p) {
  const unsigned long long m = __ballot(p);
  return m ? 63 - __builtin_clzll(m) : -1;
}
__device__ inline float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ inline int lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// (value, index) argmax over the wave: larger value, then lower index.
__device__ inline void am_step(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ inline void seg_reduce_am(int S, float& v, int& i) {
  if (S >= 2) am_step(v, i, dpp_f<kDppXor1>(v), dpp_i<kDppXor1>(i));
  if (S >= 4) am_step(v, i, dpp_f<kDppXor2>(v), dpp_i<kDppXor2>(i));
  if (S >= 8) am_step(v, i, dpp_f<kDppHalfMirror>(v), dpp_i<kDppHalfMirror>(i));
  if (S >= 16) am_step(v, i, dpp_f<kDppMirror>(v), dpp_i<kDppMirror>(i));
  if (S >= 32) am_step(v, i, __shfl_xor(v, 16), __shfl_xor(i, 16));
  if (S >= 64) am_step(v, i, __shfl_xor(v, 32), __shfl_xor(i, 32));
}

template <int kCtrl>
__device__ inline void am_dpp(float& v, int& i) {
  const float v2 = dpp_f<kCtrl>(v);
  const int i2 = dpp_i<kCtrl>(i);
  am_step(v, i, v2, i2);
}
__device__ inline void wave_argmax_all(float& v, int& i) {
  am_dpp<kDppXor1>(v, i);
  am_dpp<kDppXor2>(v, i);
  am_dpp<kDppHalfMirror>(v, i);
  am_dpp<kDppMirror>(v, i);
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row)
    am_step(bv, bi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), row * 16)),
            __builtin_amdgcn_readlane(i, row * 16));
  v = bv;
  i = bi;
}

// Merge two (max, sum of 2^(y - max)) pairs.
__device__ inline void ms_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) { m = mn; s = 0.f; return; }
  s = s * fast_exp2(m - mn) + s2 * fast_exp2(m2 - mn);
  m = mn;
}

// Segmented reductions over aligned groups of S consecutive lanes (S a
// power of two, uniform): every lane of a group ends with its group's
// result. Within a row of 16 lanes the butterfly runs on DPP (quad
// permutes, half-row mirror, row mirror); wider groups add lane shuffles.
// Every lane of the wave must be active.
__device__ inline void seg_reduce_ms(int S, float& m, float& s) {
  float m2, s2;
  if (S >= 2) { m2 = dpp_f<kDppXor1>(m); s2 = dpp_f<kDppXor1>(s); ms_merge(m, s, m2, s2); }
  if (S >= 4) { m2 = dpp_f<kDppXor2>(m); s2 = dpp_f<kDppXor2>(s); ms_merge(m, s, m2, s2); }
  if (S >= 8) { m2 = dpp_f<kDppHalfMirror>(m); s2 = dpp_f<kDppHalfMirror>(s); ms_merge(m, s, m2, s2); }
  if (S >= 16) { m2 = dpp_f<kDppMirror>(m); s2 = dpp_f<kDppMirror>(s); ms_merge(m, s, m2, s2); }
  if (S >= 32) { m2 = __shfl_xor(m, 16); s2 = __shfl_xor(s, 16); ms_merge(m, s, m2, s2); }
  if (S >= 64) { m2 = __shfl_xor(m, 32); s2 = __shfl_xor(s, 32); ms_merge(m, s, m2, s2); }
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
