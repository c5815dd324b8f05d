// gfx950 kernels and host entry points of the speculative-decoding verifier.
//
// Design (one GPU, one stream, no host synchronisation):
//   row pass   one workgroup per (request, row, segment of V). It streams its
//              segment once with 128-bit loads and writes a partial: the
//              online-softmax pair (max, sum of 2^(y - max)) with
//              y = logit * log2(e) / T for sampling, or (max, argmax) for
//              greedy/tree. The last workgroup of a request (per-request
//              atomic ticket) merges the partials and runs that request's
//              tail: Philox uniforms, the acceptance scan, and the draw.
//   draw       the draw needs only the partials plus ONE re-read segment:
//              the segment sums locate the segment that holds u * Z, and a
//              workgroup scan inside it finds the token. With one-hot
//              drafts the row pass already leaves the draft token out of
//              its row's sums, so the residual max(0, p - onehot) costs no
//              extra pass.
//   residual   (explicit draft logits only) the residual max(0, p_a - q_a)
//   pass       needs the normalisers of both rows, so a second launch
//              streams the stop rows of the rejected requests in segments
//              and its last workgroup per request draws the token.
// The rule follows "【大模型基础设施工程】15：推测解码与 MTP" §2.1 (accept x_i
// with probability min(1, p_i(x_i)/q_i(x_i)); on the first rejection draw
// from the normalised max(0, p_i - q_i) and stop; bonus from the last
// row when all are accepted), §3.3 (tree) and §11 (greedy).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "specverify.h"
#include "sv_device.hpp"

namespace sv {

enum Mode { kOneHot = 0, kExplicit = 1, kGreedy = 2, kTree = 3 };

constexpr int kMaxRows = 2 * SV_MAX_DRAFT + 1;
constexpr size_t kCounterBytes = 4u * SV_MAX_BATCH;
constexpr int kSegMin = 2048;             // smallest segment any dtype uses

// Loads per thread per segment: 4 x 16 B for bf16 (8192 logits), 8 x 16 B
// for fp32 (8192 logits): 16 / 32 KiB per workgroup.
constexpr int kUBf16 = 4;
constexpr int kUF32 = 8;

// Hand-off from the row pass to the residual pass (explicit draft logits).
struct Record {
  int a;          // stop position
  int pending;    // 1: the residual draw is still to be done
  float c;        // log2(e) / T
  float u;        // sampling uniform of position a
  float Mp, Sp;   // target row a: max and sum in units of 2^(y - Mp)
  float Mq, Sq;   // draft row a
};

struct Args {
  const char* tgt; int64_t t_sb, t_sk;     // byte strides
  const char* drf; int64_t d_sb, d_sk;
  const int32_t* tokens;                   // [B, K] drafts or [B, N] node tokens
  const float* temperature;                // [B]
  const uint64_t* seeds;                   // [B]
  uint64_t offset;
  int B, K, V;
  int R;          // target rows per request
  int rows;       // rows per request in the row pass (target + draft)
  int n_seg;      // segments per row
  int out_cols;   // row length of out_tokens
  int32_t* out_tokens; int32_t* out_len; float* out_p; float* out_q; int32_t* out_aux;
  unsigned* counters;   // [B], zero between calls
  float2* part;         // [B * rows * n_seg]
  Record* rec;          // [B]
  float* res_part;      // [B * n_seg]
  int n_nodes;
  int8_t parent[SV_MAX_TREE_NODES];
};

struct TailLds {
  float red[kWaves];
  float red2[kWaves];
  int red_i[kWaves];
  int imin, imax, a, found;
  float tin;
  float rowM[kMaxRows], rowS[kMaxRows];
  float selM[SV_MAX_DRAFT + 1], selZ[SV_MAX_DRAFT + 1];
  float p[SV_MAX_DRAFT + 1], q[SV_MAX_DRAFT + 1];
  float uacc[SV_MAX_DRAFT + 1], usmp[SV_MAX_DRAFT + 1];
  int x[SV_MAX_TREE_NODES], g[SV_MAX_TREE_NODES], path[SV_MAX_TREE_NODES];
  int depth[SV_MAX_TREE_NODES];
};

__device__ inline const char* row_ptr(const Args& A, int b, int r) {
  return r < A.R ? A.tgt + (int64_t)b * A.t_sb + (int64_t)r * A.t_sk
                 : A.drf + (int64_t)b * A.d_sb + (int64_t)(r - A.R) * A.d_sk;
}

// ------------------------------------------------------------ drawing ---
// Which segment holds the draw: Z = sum_s W(s), t = u * Z, first s whose
// running sum exceeds t. Leaves S.found = segment (or the last segment of
// positive weight when rounding leaves none, with S.tin = +inf) and
// S.tin = t minus the weight before it. Returns Z.
template <class WFn>
__device__ float locate_segment(int n_seg, float u, WFn W, TailLds& S) {
  const int tid = threadIdx.x;
  float Z = 0.f;
  for (int base = 0; base < n_seg; base += kThreads) {
    const int s = base + tid;
    Z += block_sum(s < n_seg ? W(s) : 0.f, S.red);
  }
  const float t = u * Z;
  if (tid == 0) { S.imin = INT_MAX; S.imax = -1; }
  __syncthreads();
  float carry = 0.f;
  for (int base = 0; base < n_seg; base += kThreads) {
    const int s = base + tid;
    const float w = s < n_seg ? W(s) : 0.f;
    float tot;
    const float incl = carry + block_incl_scan(w, S.red, tot);
    if (s < n_seg && incl > t && w > 0.f) atomicMin(&S.imin, s);
    if (s < n_seg && w > 0.f) atomicMax(&S.imax, s);
    __syncthreads();
    const int hit = S.imin;
    if (hit != INT_MAX) {
      if (s == hit) S.tin = t - (incl - w);
      break;
    }
    carry += tot;
  }
  __syncthreads();
  if (tid == 0) {
    if (S.imin != INT_MAX) {
      S.found = S.imin;
    } else {
      S.found = S.imax;                 // rounding overshoot: last positive segment
      S.tin = __builtin_inff();
    }
  }
  __syncthreads();
  return Z;
}

// Inside one segment: the smallest element whose running weight sum
// exceeds t_in, scanning vectors in index order (vector j of thread t is
// the (j * kThreads + t)-th of the segment); the last element of positive
// weight if rounding leaves none.
template <int kPer, int U>
__device__ int pick_in_segment(const float (&w)[U * kPer], int64_t seg0, float t_in, TailLds& S) {
  const int tid = threadIdx.x;
  if (tid == 0) { S.imin = INT_MAX; S.imax = -1; }
  __syncthreads();
  float carry = 0.f;
  for (int j = 0; j < U; ++j) {
    float vs = 0.f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) vs += w[j * kPer + k];
    float tot;
    const float incl = carry + block_incl_scan(vs, S.red, tot);
    const int e0 = (int)(seg0 + (int64_t)(j * kThreads + tid) * kPer);
    if (incl > t_in) {
      float run = incl - vs;
      int hit = -1;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        run += w[j * kPer + k];
        if (hit < 0 && run > t_in && w[j * kPer + k] > 0.f) hit = k;
      }
      if (hit >= 0) atomicMin(&S.imin, e0 + hit);
    }
    int last = -1;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (w[j * kPer + k] > 0.f) last = e0 + k;
    if (last >= 0) atomicMax(&S.imax, last);
    __syncthreads();
    if (S.imin != INT_MAX) break;
    carry += tot;
  }
  __syncthreads();
  const int y = S.imin != INT_MAX ? S.imin : S.imax;
  __syncthreads();
  return y;
}

// Draw from one row's softmax weights 2^(y - M) (optionally without token
// `xe`) using that row's row-pass partials; used for the one-hot residual
// and the bonus token. Returns -1 when the weights have no mass.
template <int DT, int U, bool kVec>
__device__ int draw_softmax_row(const Args& A, int b, int r, float c, float M, int xe, float u,
                                TailLds& S) {
  constexpr int kPer = Elem<DT>::kPerVec, kLen = kThreads * U * kPer;
  const float2* pr = A.part + ((int64_t)b * A.rows + r) * A.n_seg;
  auto W = [&](int s) {
    const float2 v = pr[s];
    return v.x == kNegInf ? 0.f : v.y * fast_exp2(v.x - M);
  };
  const float Z = locate_segment(A.n_seg, u, W, S);
  if (!(Z > 0.f) || S.found < 0) return -1;
  const int seg = S.found;
  const float t_in = S.tin;
  const int64_t seg0 = (int64_t)seg * kLen;
  float x[U * kPer];
  load_segment<DT, U, kVec>(row_ptr(A, b, r), seg0, A.V, x);
  float w[U * kPer];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t e0 = seg0 + (int64_t)(j * kThreads + threadIdx.x) * kPer;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float v = fast_exp2(fmaf(x[j * kPer + k], c, -M));
      w[j * kPer + k] = (e0 + k == xe) ? 0.f : v;
    }
  }
  return pick_in_segment<kPer, U>(w, seg0, t_in, S);
}

// ---------------------------------------------------------- row tails ---
template <int DT, int U, bool kVec, int MODE>
__device__ void sample_tail(const Args& A, int b, TailLds& S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = A.K, V = A.V, R = A.R;
  for (int rr = wave; rr < A.rows; rr += kWaves) {
    float m = kNegInf, s = 0.f;
    const float2* pr = A.part + ((int64_t)b * A.rows + rr) * A.n_seg;
    for (int sg = lane; sg < A.n_seg; sg += 64) {
      const float2 v = pr[sg];
      ms_merge(m, s, v.x, v.y);
    }
    wave_reduce_ms(m, s);
    if (lane == 0) { S.rowM[rr] = m; S.rowS[rr] = s; }
  }
  const float T = A.temperature[b];
  const bool ok = T > 0.f && T < __builtin_inff();
  const float c = kLog2e / T;
  int32_t* otok = A.out_tokens + (int64_t)b * A.out_cols;
  __syncthreads();
  if (!ok) {                                  // refused request
    if (tid <= K) otok[tid] = -1;
    if (tid < K && A.out_p) A.out_p[(int64_t)b * K + tid] = 0.f;
    if (tid < K && A.out_q) A.out_q[(int64_t)b * K + tid] = 0.f;
    if (tid == 0) {
      A.out_len[b] = 0;
      if (MODE == kExplicit) A.rec[b].pending = 0;
    }
    return;
  }
  if (tid <= K) {
    const int i = tid;
    const Philox4 rnd = philox4x64_10((uint64_t)i, (uint64_t)b, A.offset, 0ull, A.seeds[b], 0ull);
    S.uacc[i] = top24(rnd.w0);
    S.usmp[i] = top24(rnd.w1);
    if (i < K) {
      const int x = A.tokens[(int64_t)b * K + i];
      S.x[i] = x;
      const bool valid = (unsigned)x < (unsigned)V;
      const float lx = valid ? load_one<DT>(row_ptr(A, b, i), x) : kNegInf;
      float p, q;
      if (MODE == kOneHot) {
        // row-pass sums of row i leave x out: add its own term back for p(x)
        const float Mi = S.rowM[i], Si = S.rowS[i];
        const float Mn = fmaxf(Mi, lx * c);
        const float Sx = (Mi == kNegInf) ? 0.f : Si * fast_exp2(Mi - Mn);
        const float e = (valid && Mn != kNegInf) ? fast_exp2(fmaf(lx, c, -Mn)) : 0.f;
        const float St = Sx + e;
        p = St > 0.f ? e / St : 0.f;
        q = valid ? 1.f : 0.f;
        S.selM[i] = Mn;
        S.selZ[i] = Sx;
      } else {
        const float Mp = S.rowM[i], Sp = S.rowS[i];
        const float Mq = S.rowM[R + i], Sq = S.rowS[R + i];
        const float ld = valid ? load_one<DT>(row_ptr(A, b, R + i), x) : kNegInf;
        p = (valid && Sp > 0.f) ? fast_exp2(fmaf(lx, c, -Mp)) / Sp : 0.f;
        q = (valid && Sq > 0.f) ? fast_exp2(fmaf(ld, c, -Mq)) / Sq : 0.f;
      }
      S.p[i] = p;
      S.q[i] = q;
      if (A.out_p) A.out_p[(int64_t)b * K + i] = p;
      if (A.out_q) A.out_q[(int64_t)b * K + i] = q;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    while (a < K && S.uacc[a] * S.q[a] < S.p[a]) ++a;
    S.a = a;
  }
  __syncthreads();
  const int a = S.a;
  if (tid <= K && tid != a) otok[tid] = tid < a ? S.x[tid] : -1;
  if (tid == 0) A.out_len[b] = a + 1;
  if (MODE == kExplicit) {
    if (a < K) {
      if (tid == 0) {
        Record rc;
        rc.a = a; rc.pending = 1; rc.c = c; rc.u = S.usmp[a];
        rc.Mp = S.rowM[a]; rc.Sp = S.rowS[a]; rc.Mq = S.rowM[R + a]; rc.Sq = S.rowS[R + a];
        A.rec[b] = rc;
      }
      return;
    }
    if (tid == 0) A.rec[b].pending = 0;
  }
  const bool resid = (MODE == kOneHot && a < K);
  const float M = resid ? S.selM[a] : S.rowM[a];
  const int xe = resid ? S.x[a] : -1;
  int y = draw_softmax_row<DT, U, kVec>(A, b, a, c, M, xe, S.usmp[a], S);
  if (y < 0) y = ((unsigned)xe < (unsigned)V) ? xe : 0;    // residual without mass: p_a's mode
  if (tid == 0) otok[a] = y;
}

__device__ inline void merge_argmax_rows(const Args& A, int b, int n_rows, TailLds& S) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int rr = wave; rr < n_rows; rr += kWaves) {
    float v = kNegInf;
    int idx = INT_MAX;
    const float2* pr = A.part + ((int64_t)b * A.rows + rr) * A.n_seg;
    for (int sg = lane; sg < A.n_seg; sg += 64) {
      const float2 t = pr[sg];
      am_merge(v, idx, t.x, __float_as_int(t.y));
    }
    wave_reduce_am(v, idx);
    if (lane == 0) S.g[rr] = idx;
  }
}

__device__ void greedy_tail(const Args& A, int b, TailLds& S) {
  const int tid = threadIdx.x, K = A.K;
  merge_argmax_rows(A, b, A.rows, S);
  if (tid < K) S.x[tid] = A.tokens[(int64_t)b * K + tid];
  __syncthreads();
  if (tid == 0) {
    int a = 0;
    while (a < K && S.x[a] == S.g[a]) ++a;
    S.a = a;
    A.out_len[b] = a + 1;
  }
  __syncthreads();
  const int a = S.a;
  if (tid <= K) {
    A.out_tokens[(int64_t)b * A.out_cols + tid] = tid < a ? S.x[tid] : (tid == a ? S.g[a] : -1);
    if (A.out_aux) A.out_aux[(int64_t)b * (K + 1) + tid] = S.g[tid];
  }
}

__device__ void tree_tail(const Args& A, int b, TailLds& S) {
  const int tid = threadIdx.x, N = A.n_nodes;
  merge_argmax_rows(A, b, N, S);
  if (tid < N) S.x[tid] = A.tokens[(int64_t)b * N + tid];
  __syncthreads();
  if (tid == 0) {
    uint64_t acc = 1ull;
    int best = 0;
    S.depth[0] = 0;
    for (int n = 1; n < N; ++n) {
      const int p = A.parent[n];
      S.depth[n] = S.depth[p] + 1;
      if (((acc >> p) & 1ull) && S.x[n] == S.g[p]) {
        acc |= 1ull << n;
        if (S.depth[n] > S.depth[best]) best = n;
      }
    }
    const int len = S.depth[best];
    int n = best;
    for (int pos = len - 1; pos >= 0; --pos) {
      S.path[pos] = S.x[n];
      n = A.parent[n];
    }
    S.path[len] = S.g[best];
    S.a = len;
    A.out_len[b] = len + 1;
    if (A.out_aux) A.out_aux[b] = best;
  }
  __syncthreads();
  if (tid < N) A.out_tokens[(int64_t)b * A.out_cols + tid] = tid <= S.a ? S.path[tid] : -1;
}

// ------------------------------------------------------------ row pass ---
template <int MODE, int DT, int U, bool kVec>
__global__ __launch_bounds__(kThreads) void sv_rows_kernel(Args A) {
  constexpr int kPer = Elem<DT>::kPerVec, kLen = kThreads * U * kPer;
  __shared__ TailLds S;
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = (int)(blockIdx.x % (unsigned)A.n_seg);
  const int rowg = (int)(blockIdx.x / (unsigned)A.n_seg);
  const int b = rowg / A.rows, r = rowg % A.rows;
  const int64_t seg0 = (int64_t)seg * kLen;

  float x[U * kPer];
  load_segment<DT, U, kVec>(row_ptr(A, b, r), seg0, A.V, x);

  float2 res;
  if constexpr (MODE == kOneHot || MODE == kExplicit) {
    if (MODE == kOneHot && r < A.K) {
      // one-hot residual: this row's sums leave the draft token out
      const int xe = A.tokens[(int64_t)b * A.K + r];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int64_t d = (int64_t)xe - (seg0 + (int64_t)(j * kThreads + tid) * kPer);
        if (d >= 0 && d < kPer) {
#pragma unroll
          for (int k = 0; k < kPer; ++k)
            if (k == d) x[j * kPer + k] = kNegInf;
        }
      }
    }
    const float c = kLog2e / A.temperature[b];
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < U * kPer; ++e) mx = fmaxf(mx, x[e]);
    const float msub = (mx == kNegInf) ? 0.f : mx * c;
    float acc[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      acc[j] = 0.f;
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc[j] += fast_exp2(fmaf(x[j * kPer + k], c, -msub));
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < U; ++j) s += acc[j];
    float m = (mx == kNegInf) ? kNegInf : msub;
    wave_reduce_ms(m, s);
    if (lane == 0) { S.red[wave] = m; S.red2[wave] = s; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kWaves; ++w) ms_merge(m, s, S.red[w], S.red2[w]);
      res = make_float2(m, s);
    }
  } else {
    float best = x[0];
    int bi = (int)(seg0 + (int64_t)tid * kPer);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int e0 = (int)(seg0 + (int64_t)(j * kThreads + tid) * kPer);
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (x[j * kPer + k] > best) { best = x[j * kPer + k]; bi = e0 + k; }
    }
    wave_reduce_am(best, bi);
    if (lane == 0) { S.red[wave] = best; S.red_i[wave] = bi; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kWaves; ++w) am_merge(best, bi, S.red[w], S.red_i[w]);
      res = make_float2(best, __int_as_float(bi));
    }
  }

  if (tid == 0) {
    A.part[(int64_t)rowg * A.n_seg + seg] = res;
    __threadfence();                              // publish the partial ...
    const unsigned prev = atomicAdd(&A.counters[b], 1u);   // ... then take a ticket
    s_last = (prev == (unsigned)(A.rows * A.n_seg - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();                                // see every partial of request b
  if (tid == 0) A.counters[b] = 0u;               // clean for the next call
  if constexpr (MODE == kOneHot || MODE == kExplicit) {
    sample_tail<DT, U, kVec, MODE>(A, b, S);
  } else if constexpr (MODE == kGreedy) {
    greedy_tail(A, b, S);
  } else {
    tree_tail(A, b, S);
  }
}

// ------------------------------------------------------ residual pass ---
// Explicit draft logits: for requests that stopped at a < K, segment sums of
// max(0, p_a - q_a); the last workgroup of the request draws the token.
template <int DT, int U, bool kVec>
__global__ __launch_bounds__(kThreads) void sv_residual_kernel(Args A) {
  constexpr int kPer = Elem<DT>::kPerVec, kLen = kThreads * U * kPer;
  __shared__ TailLds S;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int seg = (int)(blockIdx.x % (unsigned)A.n_seg);
  const int b = (int)(blockIdx.x / (unsigned)A.n_seg);
  const Record rc = A.rec[b];
  if (!rc.pending) return;
  const int a = rc.a;
  const float c = rc.c;
  const float ip = 1.f / rc.Sp, iq = 1.f / rc.Sq;
  const char* rowp = row_ptr(A, b, a);
  const char* rowq = row_ptr(A, b, A.R + a);
  const int64_t seg0 = (int64_t)seg * kLen;

  float xp[U * kPer], xq[U * kPer];
  load_segment<DT, U, kVec>(rowp, seg0, A.V, xp);
  load_segment<DT, U, kVec>(rowq, seg0, A.V, xq);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < U * kPer; ++e)
    s += fmaxf(fast_exp2(fmaf(xp[e], c, -rc.Mp)) * ip - fast_exp2(fmaf(xq[e], c, -rc.Mq)) * iq, 0.f);
  s = block_sum(s, S.red);
  if (tid == 0) {
    A.res_part[(int64_t)b * A.n_seg + seg] = s;
    __threadfence();
    const unsigned prev = atomicAdd(&A.counters[b], 1u);
    s_last = (prev == (unsigned)(A.n_seg - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid == 0) A.counters[b] = 0u;

  const float* rp = A.res_part + (int64_t)b * A.n_seg;
  auto W = [&](int sg) { return rp[sg]; };
  const float Z = locate_segment(A.n_seg, rc.u, W, S);
  int y;
  if (Z > 0.f && S.found >= 0) {
    const int fs = S.found;
    const float t_in = S.tin;
    const int64_t f0 = (int64_t)fs * kLen;
    load_segment<DT, U, kVec>(rowp, f0, A.V, xp);
    load_segment<DT, U, kVec>(rowq, f0, A.V, xq);
    float w[U * kPer];
#pragma unroll
    for (int e = 0; e < U * kPer; ++e)
      w[e] = fmaxf(fast_exp2(fmaf(xp[e], c, -rc.Mp)) * ip - fast_exp2(fmaf(xq[e], c, -rc.Mq)) * iq, 0.f);
    y = pick_in_segment<kPer, U>(w, f0, t_in, S);
  } else {
    // p_a and q_a agree everywhere: draw from p_a
    y = draw_softmax_row<DT, U, kVec>(A, b, a, c, rc.Mp, -1, rc.u, S);
    if (y < 0) y = 0;
  }
  if (tid == 0) A.out_tokens[(int64_t)b * A.out_cols + a] = y;
}

__global__ void sv_zero_kernel(unsigned char* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (((uintptr_t)p & 3u) == 0) {
    uint32_t* w = reinterpret_cast<uint32_t*>(p);
    const size_t nw = n / 4;
    for (size_t i = i0; i < nw; i += stride) w[i] = 0u;
    for (size_t i = nw * 4 + i0; i < n; i += stride) p[i] = 0;
  } else {
    for (size_t i = i0; i < n; i += stride) p[i] = 0;
  }
}

}  // namespace sv

// ================================================================ host ===
namespace {

using namespace sv;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t part, rec, res, total;
};

// Workspace: [counters: 4 * SV_MAX_BATCH][partials][records][residual partials]
Layout layout(int64_t B, int64_t rows, int64_t V) {
  const int64_t nseg = (V + kSegMin - 1) / kSegMin;
  Layout L;
  L.part = align_up(kCounterBytes, 256);
  L.rec = align_up(L.part + (size_t)(B * rows * nseg) * sizeof(float2), 256);
  L.res = align_up(L.rec + (size_t)B * sizeof(Record), 256);
  L.total = align_up(L.res + (size_t)(B * nseg) * sizeof(float), 256);
  return L;
}

int elem_bytes(int dtype) { return dtype == SV_DTYPE_BF16 ? 2 : 4; }

int seg_len(int dtype) {
  return dtype == SV_DTYPE_BF16 ? kThreads * kUBf16 * Elem<kBF16>::kPerVec
                                : kThreads * kUF32 * Elem<kF32>::kPerVec;
}

int check_desc(const sv_logits* d) {
  if (!d || !d->data) return SV_ERR_NULL;
  if ((d->dtype != SV_DTYPE_F32 && d->dtype != SV_DTYPE_BF16) || d->reserved != 0)
    return SV_ERR_DTYPE;
  if (d->stride_b < 0 || d->stride_k < 0) return SV_ERR_STRIDE;
  return SV_OK;
}

bool aligned16(const sv_logits* d) {
  const int64_t es = elem_bytes(d->dtype);
  return ((uintptr_t)d->data % 16 == 0) && ((d->stride_b * es) % 16 == 0) &&
         ((d->stride_k * es) % 16 == 0);
}

void fill_common(Args& A, const sv_logits* t, int B, int K, int V, int R, int rows,
                 void* ws, int dtype) {
  const int64_t es = elem_bytes(dtype);
  A.tgt = static_cast<const char*>(t->data);
  A.t_sb = t->stride_b * es;
  A.t_sk = t->stride_k * es;
  A.drf = nullptr; A.d_sb = 0; A.d_sk = 0;
  A.B = B; A.K = K; A.V = V; A.R = R; A.rows = rows;
  A.n_seg = (V + seg_len(dtype) - 1) / seg_len(dtype);
  const Layout L = layout(B, rows, V);
  unsigned char* base = static_cast<unsigned char*>(ws);
  A.counters = reinterpret_cast<unsigned*>(base);
  A.part = reinterpret_cast<float2*>(base + L.part);
  A.rec = reinterpret_cast<Record*>(base + L.rec);
  A.res_part = reinterpret_cast<float*>(base + L.res);
  A.out_p = nullptr; A.out_q = nullptr; A.out_aux = nullptr;
  A.temperature = nullptr; A.seeds = nullptr; A.offset = 0;
  A.n_nodes = 0;
  for (int i = 0; i < SV_MAX_TREE_NODES; ++i) A.parent[i] = -1;
}

#define SV_LAUNCH(KERNEL, grid, st, A) \
  hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(kThreads), 0, st, A)

template <int MODE>
void launch_rows(const Args& A, int dtype, bool vec, unsigned grid, hipStream_t st) {
  if (dtype == SV_DTYPE_BF16) {
    if (vec) SV_LAUNCH((sv_rows_kernel<MODE, kBF16, kUBf16, true>), grid, st, A);
    else     SV_LAUNCH((sv_rows_kernel<MODE, kBF16, kUBf16, false>), grid, st, A);
  } else {
    if (vec) SV_LAUNCH((sv_rows_kernel<MODE, kF32, kUF32, true>), grid, st, A);
    else     SV_LAUNCH((sv_rows_kernel<MODE, kF32, kUF32, false>), grid, st, A);
  }
}

void launch_residual(const Args& A, int dtype, bool vec, unsigned grid, hipStream_t st) {
  if (dtype == SV_DTYPE_BF16) {
    if (vec) SV_LAUNCH((sv_residual_kernel<kBF16, kUBf16, true>), grid, st, A);
    else     SV_LAUNCH((sv_residual_kernel<kBF16, kUBf16, false>), grid, st, A);
  } else {
    if (vec) SV_LAUNCH((sv_residual_kernel<kF32, kUF32, true>), grid, st, A);
    else     SV_LAUNCH((sv_residual_kernel<kF32, kUF32, false>), grid, st, A);
  }
}

// A dispatch counts work-items in 32 bits per dimension.
int check_grid(int64_t wgs) {
  return (wgs >= 1 && wgs <= (int64_t)(UINT32_MAX / kThreads)) ? SV_OK : SV_ERR_SHAPE;
}

int hip_status() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP; }

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int32_t op, int32_t B, int32_t K_or_N, int32_t V,
                                  int32_t has_draft) {
  if (B < 1 || B > SV_MAX_BATCH || V < 1 || V > SV_MAX_VOCAB) return 0;
  int64_t rows;
  if (op == SV_OP_SAMPLE) {
    if (K_or_N < 0 || K_or_N > SV_MAX_DRAFT) return 0;
    rows = (int64_t)K_or_N + 1 + (has_draft ? K_or_N : 0);
  } else if (op == SV_OP_GREEDY) {
    if (K_or_N < 0 || K_or_N > SV_MAX_DRAFT) return 0;
    rows = (int64_t)K_or_N + 1;
  } else if (op == SV_OP_TREE) {
    if (K_or_N < 2 || K_or_N > SV_MAX_TREE_NODES) return 0;
    rows = K_or_N;
  } else {
    return 0;
  }
  return layout(B, rows, V).total;
}

int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return SV_ERR_NULL;
  if (workspace_bytes == 0) return SV_OK;
  size_t blocks = (workspace_bytes / 4 + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(sv_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<unsigned char*>(workspace), workspace_bytes);
  return hip_status();
}

int spec_verify_sample(const sv_logits* target, const sv_logits* draft,
                       const int32_t* draft_tokens, const float* temperature,
                       const uint64_t* seeds, uint64_t offset,
                       int32_t B, int32_t K, int32_t V,
                       int32_t* out_tokens, int32_t* out_accept_len,
                       float* out_p_draft, float* out_q_draft,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(target);
  if (st) return st;
  if (draft && (st = check_desc(draft))) return st;
  if (!temperature || !seeds || !out_tokens || !out_accept_len) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_DRAFT || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if (K > 0 && !draft_tokens) return SV_ERR_NULL;
  if (draft && draft->dtype != target->dtype) return SV_ERR_DTYPE;
  if (!workspace) return SV_ERR_WORKSPACE;
  const bool explicit_q = draft != nullptr && K > 0;
  const int R = K + 1;
  const int rows = R + (explicit_q ? K : 0);
  if (workspace_bytes < layout(B, rows, V).total) return SV_ERR_WORKSPACE;

  Args A;
  fill_common(A, target, B, K, V, R, rows, workspace, target->dtype);
  if (explicit_q) {
    const int64_t es = elem_bytes(draft->dtype);
    A.drf = static_cast<const char*>(draft->data);
    A.d_sb = draft->stride_b * es;
    A.d_sk = draft->stride_k * es;
  }
  A.tokens = draft_tokens;
  A.temperature = temperature;
  A.seeds = seeds;
  A.offset = offset;
  A.out_cols = K + 1;
  A.out_tokens = out_tokens;
  A.out_len = out_accept_len;
  A.out_p = out_p_draft;
  A.out_q = out_q_draft;
  const int64_t wgs = (int64_t)B * rows * A.n_seg;
  if ((st = check_grid(wgs))) return st;
  const bool vec = aligned16(target) && (!explicit_q || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (explicit_q) {
    launch_rows<kExplicit>(A, target->dtype, vec, (unsigned)wgs, s);
    if ((st = hip_status())) return st;
    launch_residual(A, target->dtype, vec, (unsigned)((int64_t)B * A.n_seg), s);
  } else {
    launch_rows<kOneHot>(A, target->dtype, vec, (unsigned)wgs, s);
  }
  return hip_status();
}

int spec_verify_greedy(const sv_logits* target, const int32_t* draft_tokens,
                       int32_t B, int32_t K, int32_t V,
                       int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(target);
  if (st) return st;
  if (!out_tokens || !out_accept_len) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_DRAFT || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if (K > 0 && !draft_tokens) return SV_ERR_NULL;
  if (!workspace) return SV_ERR_WORKSPACE;
  const int R = K + 1;
  if (workspace_bytes < layout(B, R, V).total) return SV_ERR_WORKSPACE;
  Args A;
  fill_common(A, target, B, K, V, R, R, workspace, target->dtype);
  A.tokens = draft_tokens;
  A.out_cols = K + 1;
  A.out_tokens = out_tokens;
  A.out_len = out_accept_len;
  A.out_aux = out_argmax;
  const int64_t wgs = (int64_t)B * R * A.n_seg;
  if ((st = check_grid(wgs))) return st;
  launch_rows<kGreedy>(A, target->dtype, aligned16(target), (unsigned)wgs,
                       static_cast<hipStream_t>(stream));
  return hip_status();
}

int spec_verify_tree(const sv_logits* target, const int32_t* node_tokens,
                     const int32_t* parents, int32_t N, int32_t B, int32_t V,
                     int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_best_node,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(target);
  if (st) return st;
  if (!node_tokens || !parents || !out_tokens || !out_accept_len) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || V < 1 || V > SV_MAX_VOCAB || N < 2 || N > SV_MAX_TREE_NODES)
    return SV_ERR_SHAPE;
  if (parents[0] != -1) return SV_ERR_TREE;
  for (int n = 1; n < N; ++n)
    if (parents[n] < 0 || parents[n] >= n) return SV_ERR_TREE;
  if (!workspace) return SV_ERR_WORKSPACE;
  if (workspace_bytes < layout(B, N, V).total) return SV_ERR_WORKSPACE;
  Args A;
  fill_common(A, target, B, 0, V, N, N, workspace, target->dtype);
  A.tokens = node_tokens;
  A.out_cols = N;
  A.out_tokens = out_tokens;
  A.out_len = out_accept_len;
  A.out_aux = out_best_node;
  A.n_nodes = N;
  for (int n = 0; n < N; ++n) A.parent[n] = (int8_t)parents[n];
  const int64_t wgs = (int64_t)B * N * A.n_seg;
  if ((st = check_grid(wgs))) return st;
  launch_rows<kTree>(A, target->dtype, aligned16(target), (unsigned)wgs,
                     static_cast<hipStream_t>(stream));
  return hip_status();
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "batch, draft count, node count or vocabulary out of range";
    case SV_ERR_DTYPE: return "unknown logits dtype, nonzero reserved field, or draft dtype differs";
    case SV_ERR_STRIDE: return "negative logits stride";
    case SV_ERR_WORKSPACE: return "workspace missing or smaller than spec_verify_workspace_size()";
    case SV_ERR_TREE: return "malformed parent array (need parents[0] == -1, 0 <= parents[n] < n)";
    case SV_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
