// gfx950 kernels and host entry points of the speculative-decoding verifier.
//
// Design (one GPU, one stream, no host synchronisation):
//   row pass   the logits of every (request, row) are cut into 4 KiB chunks
//              (2048 bf16 or 1024 fp32 logits). A workgroup owns a run of
//              chunks of one row; each of its four waves streams chunks
//              with 128-bit loads, the next chunk always in flight while
//              the current one is reduced, and writes one partial per
//              chunk: the online-softmax pair (max, sum of 2^(y - max))
//              with y = logit * log2(e) / T for sampling, or (max, argmax)
//              for greedy/tree. It also keeps the logit of each row's draft
//              token.
//   tail       one wave per request merges that request's partials and
//              runs the rule: the acceptance scan and the draw (the row
//              pass draws the Philox uniforms). Greedy, tree and one-hot
//              calls run it in the same launch: one tail workgroup per
//              request after the row pass's workgroups in the grid, fed
//              through tagged slots (see the one-launch hand-off below).
//              With draft logits the residual pass's workgroups run it.
//              Otherwise (shapes the one-launch tail cannot hold) it is a
//              second launch, and the launch boundary is the only
//              synchronisation.
//   draw       the chunk sums locate the chunk that holds u * Z, and one
//              workgroup scan over that single re-read chunk finds the
//              token. With one-hot drafts the row pass already leaves the
//              draft token out of its row's sums, so the residual
//              max(0, p - onehot) costs no extra pass.
//   residual   (explicit draft logits only) the residual max(0, p_a - q_a)
//   pass       needs the normalisers of both rows, so a third launch
//              streams the stop rows of the rejected requests in chunks;
//              the last of its workgroups per request (a per-request
//              ticket) draws the token.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "specverify.h"
#include "sv_device.hpp"

namespace sv {

enum Mode { kOneHot = 0, kExplicit = 1, kGreedy = 2, kTree = 3 };

constexpr int kMaxRows = 2 * SV_MAX_DRAFT + 1;
constexpr int kMaxChunksPerWg = 256;
constexpr size_t kHeaderBytes = 256;              // workspace header: the give-up count
constexpr size_t kCounterBytes = 4u * SV_MAX_BATCH;

// Hand-off from the row pass to the residual pass (explicit draft logits).
struct Record {
  int a;          // stop position
  int pending;    // 1: the residual draw is still to be done
  float c;        // log2(e) / T
  float u;        // sampling uniform of position a
  float Mp, Sp;   // target row a: max and sum in units of 2^(y - Mp)
  float Mq, Sq;   // draft row a
  float tp, tq;   // top-k / top-p cuts of the two rows (filtered verification)
  int draw;       // filtered verification: 1 when the token at a is still to be drawn
  int xe;         // ... leaving out this token (a one-hot draft's; -1: none)
};

// A row's top-k / top-p cut: kept logits l >= thr, weights 2^(l c - mref),
// s = their sum (without a one-hot draft token).
struct RowFilter { float mref, thr, s, pad; };

struct Args {
  const char* tgt; int64_t t_sb, t_sk;     // byte strides
  const char* drf; int64_t d_sb, d_sk;
  const int32_t* tokens;                   // [B, K] drafts or [B, N] node tokens; ragged: [total_k]
  const int32_t* cu;                       // ragged: [B + 1] prefix sums of the draft counts; else null
  int total_k;                             // ragged: number of packed drafts
  const uint32_t* mask;                    // grammar bitmask [B, K+1, mask_words] or null
  int mask_words;                          // ceil(V / 32)
  int round;                               // early-exit rounds: first position of this round, else -1
  int round_hi;                            // last position of this round
  int round_rows;                          // rows per request in a round (target + draft rows)
  int* alive;                              // [B]: request still open after the previous round
  const float* temperature;                // [B]
  const uint64_t* seeds;                   // [B]
  uint64_t offset;
  int B, K, V;
  int R;          // target rows per request
  int rows;       // rows per request in the row pass (target + draft)
  int n_chunk;    // chunks per row
  int cpw;        // chunks per workgroup
  int wpr;        // workgroups per row
  int out_cols;   // row length of out_tokens
  int32_t* out_tokens; int32_t* out_len; float* out_p; float* out_q; int32_t* out_aux;
  unsigned* counters;   // [B], zero between calls
  float2* part;         // [B * rows * n_chunk]: one partial per chunk
  float2* wpart;        // [B * rows * wpr]: one partial per row-pass workgroup
  int n_full;           // chunks per row that lie entirely below V
  float* gath;          // [B * rows]: logit of the row's draft token
  Record* rec;          // [B]
  float* res_part;      // [B * n_chunk]
  float2* unif;         // [B * R]: (u_accept, u_sample) of each position
  int filtered;         // 1: top-k / top-p filtered verification
  const int32_t* top_k; // [B] or null (no top-k)
  const float* top_p;   // [B] or null (no top-p)
  RowFilter* rf;        // [B * rows]
  float* fpart;         // [B * rows * n_chunk]: kept weight per chunk
  // one-launch calls: the row pass hands its results to tail workgroups of
  // the same grid through tagged slots (value bits, call tag), see put_tag
  uint64_t* tz_part;    // sampling: row_words words per row (run_words); argmax [B * rows * wpr][2]
  int64_t row_words;    // one-launch sampling: words per row in tz_part
  int run_block;        // one-launch sampling: words per run block in tz_part
  uint64_t* tz_gath;    // [B * rows]: logit of the row's draft token
  uint64_t* tz_unif;    // [B * R][2]: (u_accept, u_sample) of each position
  uint32_t tag;         // this call's tag
  int n_rowwg;          // row-pass workgroups; the B tail workgroups follow them in the grid
  unsigned* err;        // workspace header: count of one-launch waits that gave up
  int spin_limit;       // polls before a one-launch tail gives up
  int drop_req;         // test hook: request whose row-pass workgroups skip their tagged stores, else -1
  int no_tail;          // two-launch explicit calls: the residual pass runs the rule
  int n_nodes;
  int8_t parent[SV_MAX_TREE_NODES];
  int8_t depth[SV_MAX_TREE_NODES];   // depth of each node (root 0)
  const int32_t* dyn_parents;        // dynamic trees: [B, N] parent arrays on the device (else null)
};

// The tail keeps a request's partials in LDS when they fit, so the draw
// can locate its chunk without another trip to memory.
constexpr int kPartCache = 1024;

struct TailLds {
  float2 pcache[kPartCache];
  float rowM[kMaxRows], rowS[kMaxRows];
  int x[SV_MAX_TREE_NODES], g[SV_MAX_TREE_NODES], path[SV_MAX_TREE_NODES];
  int depth[SV_MAX_TREE_NODES];
};

// Where request b's rows, tokens and outputs are. Dense batches: K drafts
// each, rows by the two strides, tokens and p/q outputs at b * K. Ragged
// batches: K_b = cu[b + 1] - cu[b] drafts; target row i is packed row
// cu[b] + b + i and draft row i is packed row cu[b] + i (rows by stride_k),
// tokens and p/q outputs start at cu[b]. A ragged request whose offsets are
// out of order or out of range is refused and nothing of it is read.
struct Req {
  int k;          // draft count
  bool ok;
  int64_t tb;     // byte offset of target row 0
  int64_t db;     // byte offset of draft row 0
  int64_t x0;     // first draft token / p, q output
  int64_t g0;     // first argmax output (greedy)
};

__device__ inline Req request(const Args& A, int b) {
  Req q;
  if (!A.cu) {
    q.k = A.K; q.ok = true;
    q.tb = (int64_t)b * A.t_sb;
    q.db = (int64_t)b * A.d_sb;
    q.x0 = (int64_t)b * A.K;
    q.g0 = (int64_t)b * (A.K + 1);
    return q;
  }
  const int c0 = A.cu[b], c1 = A.cu[b + 1];
  q.ok = 0 <= c0 && c0 <= c1 && c1 <= A.total_k && c1 - c0 <= A.K;
  q.k = q.ok ? c1 - c0 : 0;
  const int64_t c = q.ok ? c0 : 0;
  q.tb = (c + b) * A.t_sk;
  q.db = c * A.d_sk;
  q.x0 = c;
  q.g0 = c + b;
  return q;
}

// Row r of a request: target rows first, then draft rows. Written as
// selects so that both descriptors load in one batch of scalar loads.
__device__ inline const char* row_ptr(const Args& A, const Req& q, int r) {
  const bool t = r < A.R;
  return t ? A.tgt + q.tb + (int64_t)r * A.t_sk : A.drf + q.db + (int64_t)(r - A.R) * A.d_sk;
}

// Bitmask words of position i of request b (target row i and draft row i).
__device__ inline const uint32_t* mask_row(const Args& A, int b, int i) {
  return A.mask + ((int64_t)b * A.R + i) * A.mask_words;
}

// Whether row r of a request holds data: target rows 0..k, draft rows 0..k-1.
__device__ inline bool row_live(const Args& A, const Req& q, int r) {
  return q.ok && (r < A.R ? r <= q.k : r - A.R < q.k);
}

// ------------------------------------------------ in-launch hand-off ---
// In the residual pass the workgroups of one request meet through the
// workspace inside a single launch. The L2 of each XCD is not coherent with the others, and an
// agent-scope fence writes back and invalidates a whole L2 per workgroup.
// Instead every hand-off value is written and read with device-coherent
// (relaxed agent-scope atomic, sc1) accesses that bypass the non-coherent
// cache levels; a vmcnt(0) wait makes each wave's publishes complete
// before its workgroup takes the ticket, and the ticket is a device atomic.
__device__ inline void publish(float2* p, float2 v) {
  const uint64_t bits = ((uint64_t)__float_as_uint(v.y) << 32) | __float_as_uint(v.x);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), bits, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float2 fetch(const float2* p) {
  const uint64_t bits = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)bits), __uint_as_float((uint32_t)(bits >> 32)));
}

__device__ inline float fetch(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave waits for its own publishes, then thread 0 takes the ticket:
// the count before its increment. Exactly one of the n workgroups of a
// request sees n - 1; it runs the tail and resets the counter.
__device__ inline bool last_of_request(unsigned* counter, unsigned n, int* s_last) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *s_last = (prev == n - 1);
    if (prev == n - 1) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *s_last != 0;
}

// ------------------------------------------------- one-launch hand-off ---
// Dense calls run the row pass and the per-request rule in one launch: the
// grid holds every row-pass workgroup first and then one tail workgroup per
// request. A row-pass workgroup stores its results as 64-bit words (value
// bits, tag) with device-coherent stores and ends without waiting for them;
// a tail workgroup loads the words its request needs with device-coherent
// loads until every one carries this call's tag. A 64-bit access is single-
// copy atomic, so a word with the right tag holds the right value, and a word
// left by an earlier call carries that call's tag: nothing is cleared between
// calls and no workgroup waits for its stores. Tags are negative-NaN bit
// patterns, which no other use of the workspace stores.
__device__ inline void put_tag(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t get_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline bool has_tag(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
__device__ inline float tag_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

// One-launch sampling: run wi of row rowg has a block of run_block words at
// rowg * row_words + wi * run_block: one per chunk (the chunk's sum rescaled
// to the run's largest chunk max), then that max. Blocks are whole 128-byte
// lines when the workspace has room (the host's plan): writes during the
// row pass cost per line written, far more than per byte.
__device__ inline uint64_t* run_words(const Args& A, int64_t rowg, int wi) {
  return A.tz_part + rowg * A.row_words + (int64_t)wi * A.run_block;
}

// A tail workgroup gives up after this many polls (far beyond any row pass:
// every poll is at least one trip to memory), refuses its request and
// counts the event in the workspace header, so every wave of the launch
// ends whatever the workspace holds and the caller can see that it
// happened (spec_verify_workspace_errors).
constexpr int kSpinLimit = 1 << 20;

// Tail workgroups clear every tagged word their request's row pass wrote,
// once they have seen all of them carry the call's tag: after a call that
// gave up no wait, the tagged region holds zeros only, so a word of an
// earlier call can never pass for one of a later call, whatever their tags.
__device__ inline void clear_tag(uint64_t* p) {
  __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void count_give_up(const Args& A) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(A.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Tagged words per lane a one-launch tail loads (per kind of value).
constexpr int kFusedQ = 8;

// Waits (all lanes loading one broadcast word) until the slot at p carries
// the tag: a tail first waits this way on its request's last row-pass
// workgroup, which is dispatched last and usually finishes last, and only
// then loads all its slots, so requests still streaming cost one word per
// poll instead of every slot. Returns false when the wait gave up.
__device__ inline bool wait_tag(const uint64_t* p, uint32_t tag, int limit) {
  for (int spin = 0; spin < limit; ++spin) {
    if (has_tag(get_tag(p), tag)) return true;
    __builtin_amdgcn_s_sleep(8);
  }
  return false;
}

// ------------------------------------------------------------ drawing ---
// Every draw is done by one wave: the tail of a request is short and runs
// once per request per call, so it is kept small and free of workgroup
// barriers.

// Chunk holding the draw among n chunk weights W(s): Z = sum of all, t =
// u * Z, first s whose running sum exceeds t (only chunks of positive
// weight qualify). Returns Z; *found = that chunk (or the last chunk of
// positive weight when rounding leaves none, with *t_in = +inf; -1 if no
// weight at all) and *t_in = t minus the weight before it.
template <class WFn>
__device__ __forceinline__ float wave_locate(int n, float u, WFn W, int* found, float* t_in) {
  const int lane = threadIdx.x & 63;
  if (n <= 64) {                                   // one weight per lane: a single pass
    const float w = lane < n ? W(lane) : 0.f;
    const float Z = wave_sum_all(w);
    const float t = u * Z;
    const float incl = wave_scan_incl(w);
    const int hit = first_lane(lane < n && incl > t && w > 0.f);
    if (hit >= 0) {
      *found = hit;
      *t_in = t - lane_f(incl - w, hit);
    } else {
      *found = last_lane(w > 0.f);
      *t_in = __builtin_inff();
    }
    return Z;
  }
  float Z = 0.f;
  for (int base = 0; base < n; base += 64) {
    const int s = base + lane;
    Z += wave_sum_all(s < n ? W(s) : 0.f);
  }
  const float t = u * Z;
  float carry = 0.f;
  int last = -1;
  for (int base = 0; base < n; base += 64) {
    const int s = base + lane;
    const float w = s < n ? W(s) : 0.f;
    const float incl = carry + wave_scan_incl(w);
    const int hit = first_lane(s < n && incl > t && w > 0.f);
    if (hit >= 0) {
      *found = base + hit;
      *t_in = t - lane_f(incl - w, hit);
      return Z;
    }
    const int lp = last_lane(w > 0.f);
    if (lp >= 0) last = base + lp;
    carry = lane_f(incl, 63);
  }
  *found = last;
  *t_in = __builtin_inff();
  return Z;
}

// Inside one chunk whose lane l holds the E weights of logits
// c0 + l * E ... + E - 1: the smallest logit whose running weight sum
// exceeds t_in, else the last logit of positive weight, else -1.
template <int E>
__device__ __forceinline__ int wave_pick(const float (&w)[E], int64_t c0, float t_in) {
  const int lane = threadIdx.x & 63;
  float vs = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) vs += w[k];
  float run = wave_scan_incl(vs) - vs;
  int hit = -1, last = -1;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    run += w[k];
    if (hit < 0 && run > t_in && w[k] > 0.f) hit = k;
    if (w[k] > 0.f) last = k;
  }
  const int lh = first_lane(hit >= 0);
  if (lh >= 0) return (int)(c0 + (int64_t)lh * E + lane_i(hit, lh));
  const int ll = last_lane(last >= 0);
  if (ll >= 0) return (int)(c0 + (int64_t)ll * E + lane_i(last, ll));
  return -1;
}

// Lane l's E consecutive logits c0 + l * E ... of one chunk (-inf past V).
template <int DT, bool kVec, int E>
__device__ __forceinline__ void load_lane_run(const char* row, int64_t c0, int V, float (&x)[E]) {
  constexpr int kPer = Elem<DT>::kPerVec;
  const int64_t e0 = c0 + (int64_t)(threadIdx.x & 63) * E;
  if (kVec && e0 + E <= V) {
#pragma unroll
    for (int j = 0; j < E / kPer; ++j) load_vec16<DT>(row + (e0 + j * kPer) * Elem<DT>::kBytes, &x[j * kPer]);
  } else {
#pragma unroll
    for (int k = 0; k < E; ++k) x[k] = (e0 + k < V) ? load_one<DT>(row, e0 + k) : kNegInf;
  }
}

// load_lane_run for the filtered draw: off the 16-byte path every load is
// issued (at a clamped index) before any is used, so that they are in
// flight together; logits past V then read as -inf.
template <int DT, bool kVec, int E>
__device__ __forceinline__ void load_lane_run_all(const char* row, int64_t c0, int V, float (&x)[E]) {
  constexpr int kPer = Elem<DT>::kPerVec;
  const int64_t e0 = c0 + (int64_t)(threadIdx.x & 63) * E;
  if (kVec && e0 + E <= V) {
#pragma unroll
    for (int j = 0; j < E / kPer; ++j) load_vec16<DT>(row + (e0 + j * kPer) * Elem<DT>::kBytes, &x[j * kPer]);
  } else {
#pragma unroll
    for (int k = 0; k < E; ++k) x[k] = load_one<DT>(row, min(e0 + k, (int64_t)V - 1));
#pragma unroll
    for (int k = 0; k < E; ++k) x[k] = e0 + k < V ? x[k] : kNegInf;
  }
}

// Partial (row rr of request b, chunk s), written by the row pass: from
// the tail's LDS copy when the request's partials fit there, else from the
// workspace.
__device__ inline float2 partial(const Args& A, int b, int rr, int s, const TailLds& S, bool cached) {
  return cached ? S.pcache[rr * A.n_chunk + s]
                : A.part[((int64_t)b * A.rows + rr) * A.n_chunk + s];
}

// Bitmask bits of lane l's E consecutive logits c0 + l * E ... (E = 32 or
// 16, so they sit in one word): bit k allows logit c0 + l * E + k.
template <int E>
__device__ __forceinline__ uint32_t lane_mask_bits(const uint32_t* mrow, int64_t c0, int n_words) {
  const int64_t e0 = c0 + (int64_t)(threadIdx.x & 63) * E;
  const int64_t wi = e0 >> 5;
  return mrow[wi < n_words ? wi : n_words - 1] >> (e0 & 31);
}

// Draw from one row's softmax weights 2^(y - M) (optionally without token
// `xe`) using that row's row-pass partials; used for the one-hot residual
// and the bonus token. Returns -1 when the weights have no mass.
// part_of(s) returns the row's chunk partial s. kThr: logits below thr
// weigh nothing (a top-k / top-p cut).
template <int DT, bool kVec, bool kMask, bool kThr, class PartOf>
__device__ int draw_from_partials(const Args& A, int b, const Req& rq, int r, float c, float M, int xe,
                                  float u, float thr, PartOf part_of) {
  constexpr int E = Chunk<DT>::kElems / 64;
  auto W = [&](int s) {
    const float2 v = part_of(s);
    return v.x == kNegInf ? 0.f : v.y * fast_exp2(v.x - M);
  };
  int found;
  float t_in;
  const float Z = wave_locate(A.n_chunk, u, W, &found, &t_in);
  if (!(Z > 0.f) || found < 0) return -1;
  const int64_t c0 = (int64_t)found * Chunk<DT>::kElems;
  float x[E], w[E];
  load_lane_run<DT, kVec, E>(row_ptr(A, rq, r), c0, A.V, x);
  const uint32_t allow = kMask ? lane_mask_bits<E>(mask_row(A, b, r), c0, A.mask_words) : ~0u;
  const int64_t e0 = c0 + (int64_t)(threadIdx.x & 63) * E;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const float v = fast_exp2(fmaf(x[k], c, -M));
    w[k] = (e0 + k == xe || !((allow >> k) & 1u) || (kThr && !(x[k] >= thr))) ? 0.f : v;
  }
  return wave_pick<E>(w, c0, t_in);
}

template <int DT, bool kVec, bool kMask>
__device__ int draw_softmax_row(const Args& A, int b, const Req& rq, int r, float c, float M, int xe,
                                float u, const TailLds& S, bool cached) {
  return draw_from_partials<DT, kVec, kMask, false>(A, b, rq, r, c, M, xe, u, kNegInf,
                                                     [&](int s) { return partial(A, b, r, s, S, cached); });
}

// Copying a request's partials to LDS when they fit: stage_issue starts the
// loads of the first 512 (8 per lane) so independent work can overlap
// them; stage_commit stores them, copies any rest, and syncs. Returns
// whether the partials are cached.
struct Staged { float2 v[8]; };

__device__ inline void stage_issue(const Args& A, int b, Staged& t) {
  const int lane = threadIdx.x & 63;
  const int n = A.rows * A.n_chunk;
  if (n > kPartCache) return;
  const float2* pb = A.part + (int64_t)b * n;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = q * 64 + lane;
    t.v[q] = i < n ? pb[i] : make_float2(0.f, 0.f);
  }
}

__device__ bool stage_commit(const Args& A, int b, TailLds& S, Staged& t) {
  const int lane = threadIdx.x & 63;
  const int n = A.rows * A.n_chunk;
  if (n > kPartCache) return false;
  const float2* pb = A.part + (int64_t)b * n;
  for (int base = 0; base < n; base += 8 * 64) {
    if (base) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = base + q * 64 + lane;
        t.v[q] = i < n ? pb[i] : make_float2(0.f, 0.f);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = base + q * 64 + lane;
      if (i < n) S.pcache[i] = t.v[q];
    }
  }
  __builtin_amdgcn_wave_barrier();   // one wave: order the LDS traffic
  return true;
}


// The row pass's per-workgroup partials of a request, wpr per row, loaded
// in one batch at the start of the tail: row rr's partials sit in a group
// of G lanes (G = wpr rounded up to a power of two, 64 / G rows per load,
// padded with the merge's identity), so every row merges at once with
// segmented reductions. Requests that would need more than 8 loads per
// lane merge serially from the workspace instead.
struct WStaged { float2 v[8]; int G, per, passes; };

__device__ inline void wstage_issue(const Args& A, int b, int n_rows, float2 identity, WStaged& t) {
  const int lane = threadIdx.x & 63;
  int G = 1;
  while (G < A.wpr && G < 128) G <<= 1;
  t.G = G;
  t.per = G <= 64 ? 64 / G : 0;
  t.passes = t.per > 0 ? (n_rows + t.per - 1) / t.per : 0;
  if (t.per == 0 || t.passes > 8) { t.passes = 0; return; }
  const float2* wp = A.wpart + (int64_t)b * A.rows * A.wpr;
  const int w = lane & (G - 1), rsub = lane / G;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rr = q * t.per + rsub;
    t.v[q] = identity;
    if (q < t.passes && rr < n_rows && w < A.wpr) t.v[q] = wp[rr * A.wpr + w];
  }
}

// wstage_issue's layout from tagged workgroup partials (one-launch calls):
// polls until the partials of every live row carry this call's tag. Returns
// false when the wait gave up. The host admits a one-launch call only when
// the layout fits (1 <= passes <= 8).
__device__ inline bool wstage_tagged(const Args& A, int b, int n_live, float2 identity, WStaged& t) {
  const int lane = threadIdx.x & 63;
  int G = 1;
  while (G < A.wpr) G <<= 1;
  t.G = G;
  t.per = 64 / G;
  t.passes = (A.rows + t.per - 1) / t.per;
  uint64_t* wp = A.tz_part + 2 * (int64_t)b * A.rows * A.wpr;
  const int w = lane & (G - 1), rsub = lane / G;
  uint64_t hv[8], hi[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) { hv[q] = 0ull; hi[q] = 0ull; }
  // the last live row's last workgroup first (see wait_tag)
  if (n_live > 0 && !wait_tag(wp + 2 * ((n_live - 1) * A.wpr + A.wpr - 1) + 1, A.tag, A.spin_limit))
    return false;
  for (int spin = 0;; ++spin) {
    bool miss = false;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rr = q * t.per + rsub;
      if (q < t.passes && rr < n_live && w < A.wpr) {
        const uint64_t* slot = wp + 2 * (rr * A.wpr + w);
        if (!has_tag(hv[q], A.tag)) hv[q] = get_tag(slot);
        if (!has_tag(hi[q], A.tag)) hi[q] = get_tag(slot + 1);
        miss |= !(has_tag(hv[q], A.tag) && has_tag(hi[q], A.tag));
      }
    }
    if (__ballot(miss) == 0ull) break;
    if (spin >= A.spin_limit) return false;
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rr = q * t.per + rsub;
    const bool mine = q < t.passes && rr < n_live && w < A.wpr;
    t.v[q] = mine ? make_float2(tag_val(hv[q]), tag_val(hi[q])) : identity;
  }
  return true;
}

// Clears the words wstage_tagged read (all of the call's rows, seen), for
// later calls; issued after the tail's last loads.
__device__ inline void wclear_tagged(const Args& A, int b, int n_live, const WStaged& t) {
  const int lane = threadIdx.x & 63;
  uint64_t* wp = A.tz_part + 2 * (int64_t)b * A.rows * A.wpr;
  const int w = lane & (t.G - 1), rsub = lane / t.G;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rr = q * t.per + rsub;
    if (q < t.passes && rr < n_live && w < A.wpr) {
      uint64_t* slot = wp + 2 * (rr * A.wpr + w);
      clear_tag(slot);
      clear_tag(slot + 1);
    }
  }
}

// Per-row (max, sum) into S.rowM / S.rowS.
__device__ void merge_softmax_rows(const Args& A, int b, TailLds& S, const WStaged& t) {
  const int lane = threadIdx.x & 63;
  if (t.passes > 0) {
    const int rsub = lane / t.G;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < t.passes) {                          // uniform: all lanes take part
        float m = t.v[q].x, s = t.v[q].y;
        seg_reduce_ms(t.G, m, s);
        const int rr = q * t.per + rsub;
        if ((lane & (t.G - 1)) == 0 && rr < A.rows) {
          S.rowM[rr] = m;
          S.rowS[rr] = s;
        }
      }
    }
  } else {
    const float2* wp = A.wpart + (int64_t)b * A.rows * A.wpr;
    for (int rr = lane; rr < A.rows; rr += 64) {
      float m = kNegInf, s = 0.f;
      for (int w = 0; w < A.wpr; ++w) {
        const float2 v = wp[rr * A.wpr + w];
        ms_merge(m, s, v.x, v.y);
      }
      S.rowM[rr] = m;
      S.rowS[rr] = s;
    }
  }
  __builtin_amdgcn_wave_barrier();   // one wave: order the LDS traffic
}

// Per-row argmax into sg.
__device__ void merge_argmax_rows(const Args& A, int b, int n_rows, int* sg, const WStaged& t) {
  const int lane = threadIdx.x & 63;
  if (t.passes > 0) {
    const int rsub = lane / t.G;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < t.passes) {                          // uniform: all lanes take part
        float v = t.v[q].x;
        int idx = __float_as_int(t.v[q].y);
        seg_reduce_am(t.G, v, idx);
        const int rr = q * t.per + rsub;
        if ((lane & (t.G - 1)) == 0 && rr < n_rows) sg[rr] = idx;
      }
    }
  } else {
    const float2* wp = A.wpart + (int64_t)b * A.rows * A.wpr;
    for (int rr = lane; rr < n_rows; rr += 64) {
      float v = kNegInf;
      int idx = INT_MAX;
      for (int w = 0; w < A.wpr; ++w) {
        const float2 p = wp[rr * A.wpr + w];
        am_step(v, idx, p.x, __float_as_int(p.y));
      }
      sg[rr] = idx;
    }
  }
  __builtin_amdgcn_wave_barrier();   // one wave: order the LDS traffic
}

// ---------------------------------------------------------- row tails ---
// One wave per request.
template <int DT, bool kVec, int MODE, bool kMask>
// write_out: write the outputs and the residual record (false: only return
// the decision, for the residual pass's other workgroups). Returns the
// record of a request whose residual draw is still to be done (pending 1),
// else pending 0.
__device__ Record sample_tail(const Args& A, int b, TailLds& S, bool write_out = true) {
  Record rc;
  rc.pending = 0;
  rc.draw = 0;
  rc.xe = -1;
  const int lane = threadIdx.x & 63;
  const Req rq = request(A, b);
  const int K = rq.k, V = A.V, R = A.R;
  const int64_t rowg0 = (int64_t)b * A.rows;
  // independent loads first: draft tokens, gathered logits, partials
  int x = -1;
  float lx = kNegInf, ld = kNegInf;
  if (lane < K) {
    x = A.tokens[rq.x0 + lane];
    lx = A.gath[rowg0 + lane];
    if (MODE == kExplicit) ld = A.gath[rowg0 + R + lane];
  }
  const float T = A.temperature[b];
  float2 un = make_float2(0.f, 0.f);
  if (lane <= K) un = A.unif[(int64_t)b * R + lane];
  WStaged ws;
  wstage_issue(A, b, A.rows, make_float2(kNegInf, 0.f), ws);
  Staged st;
  stage_issue(A, b, st);
  const float uacc = un.x, usmp = un.y;   // drawn by the row pass
  merge_softmax_rows(A, b, S, ws);
  const bool cached = stage_commit(A, b, S, st);
  int32_t* otok = A.out_tokens + (int64_t)b * A.out_cols;
  if (write_out)
    for (int j = K + 1 + lane; j < A.out_cols; j += 64) otok[j] = -1;   // columns past this request's drafts
  if (!rq.ok || !(T > 0.f && T < __builtin_inff())) {      // refused request
    if (!write_out) return rc;
    if (lane <= K) otok[lane] = -1;
    if (lane < K && A.out_p) A.out_p[rq.x0 + lane] = 0.f;
    if (lane < K && A.out_q) A.out_q[rq.x0 + lane] = 0.f;
    if (lane == 0) {
      A.out_len[b] = 0;
      if (MODE == kExplicit) A.rec[b].pending = 0;
    }
    return rc;
  }
  const float c = kLog2e / T;
  float p = 0.f, q = 0.f, Mx = kNegInf, lp = kNegInf, lq = kNegInf;
  if (lane < K) {
    const bool valid = (unsigned)x < (unsigned)V;
    if (!valid) { lx = kNegInf; ld = kNegInf; }
    if (MODE == kOneHot) {
      // row `lane`'s sums leave x out: add its own term back for p(x)
      const float Mi = S.rowM[lane], Si = S.rowS[lane];
      Mx = fmaxf(Mi, lx * c);
      const float Sx = (Mi == kNegInf) ? 0.f : Si * fast_exp2(Mi - Mx);
      const float e = (valid && Mx != kNegInf) ? fast_exp2(fmaf(lx, c, -Mx)) : 0.f;
      const float St = Sx + e;
      p = St > 0.f ? e / St : 0.f;
      q = valid ? 1.f : 0.f;
    } else {
      const float Mp = S.rowM[lane], Sp = S.rowS[lane];
      const float Mq = S.rowM[R + lane], Sq = S.rowS[R + lane];
      const float dp = fmaf(lx, c, -Mp), dq = fmaf(ld, c, -Mq);
      p = (valid && Sp > 0.f) ? fast_exp2(dp) / Sp : 0.f;
      q = (valid && Sq > 0.f) ? fast_exp2(dq) / Sq : 0.f;
      // log2 p and log2 q: finite where p and q underflow fp32 (both can, for
      // improbable drafts), so the test below keeps the ratio p / q
      lp = (valid && Sp > 0.f) ? dp - __log2f(Sp) : kNegInf;
      lq = (valid && Sq > 0.f) ? dq - __log2f(Sq) : kNegInf;
    }
    if (write_out && A.out_p) A.out_p[rq.x0 + lane] = p;
    if (write_out && A.out_q) A.out_q[rq.x0 + lane] = q;
  }
  // the first position whose draft is rejected (u q >= p), K if none; with
  // draft logits the test is log2 u + log2 q < log2 p (log2 0 = -inf)
  const bool accept = MODE == kOneHot ? (uacc * q < p)
                                      : (__log2f(uacc) + lq < lp);
  const int rej = first_lane(lane < K && !accept);
  const int a = rej < 0 ? K : rej;
  if (write_out) {
    if (lane <= K && lane != a) otok[lane] = lane < a ? x : -1;
    if (lane == 0) A.out_len[b] = a + 1;
  }
  const float ua = lane_f(usmp, a);
  if (MODE == kExplicit) {
    if (a < K) {
      rc.a = a; rc.pending = 1; rc.c = c; rc.u = ua;
      rc.Mp = S.rowM[a]; rc.Sp = S.rowS[a]; rc.Mq = S.rowM[R + a]; rc.Sq = S.rowS[R + a];
      rc.tp = kNegInf; rc.tq = kNegInf;
      if (write_out && lane == 0) A.rec[b] = rc;
      return rc;
    }
    if (write_out && lane == 0) A.rec[b].pending = 0;
    if (!write_out) return rc;                     // the bonus draw is the writer's
  }
  const bool resid = (MODE == kOneHot && a < K);
  const float M = resid ? lane_f(Mx, a) : S.rowM[a];
  const int xe = resid ? lane_i(x, a) : -1;
  int y = draw_softmax_row<DT, kVec, kMask>(A, b, rq, a, c, M, xe, ua, S, cached);
  if (y < 0) y = ((unsigned)xe < (unsigned)V) ? xe : 0;    // residual without mass: p_a's mode
  if (lane == 0) otok[a] = y;
  return rc;
}

// sample_tail in a one-launch call (one-hot drafts; calls with draft logits
// decide in the residual pass), spread over the tail workgroup's waves so
// that the chain after a request's last row-pass workgroup stays short:
//   wave 0  polls the request's tagged words (chunk partials of row rr,
//           chunk s in lane s % 64, load rr * npl + s / 64; the draft
//           tokens' logits; the uniforms) until all carry this call's tag,
//           hands row 0's to wave 1 through LDS as soon as they are in,
//           merges every row (max, then one rescaled sum) and runs the
//           acceptance scan; it draws itself only when the scan stops past
//           position 0;
//   wave 1  draws from row 0 as soon as its words are in: the draw of every
//           request that stops at position 0 (with one-hot drafts nearly
//           all of them) or has no drafts, made while row 1.. still stream;
//   wave 2  clears every tagged word once wave 0 has seen them all (their
//           stores in flight while the rule runs).
// The host admits a call only when rows * npl <= kFusedQ.
constexpr int kTailNotDrawn = -2;                 // wave 1 made no draw

template <int DT, bool kVec, bool kMask>
__device__ void fused_sample_tail(const Args& A, int b) {
  __shared__ float s_rowM[kFusedQ], s_rowS[kFusedQ];
  __shared__ float2 s_p0[64 * kFusedQ];            // row 0's chunk partials
  __shared__ float s_u0, s_lx0;                    // row 0's draw uniform, draft logit
  __shared__ int s_row0;                           // 0: row 0 not in yet, 1: in, 2: never
  __shared__ int s_seen;                           // 0: wave 0 still polling, 1: saw all words, 2: did not
  __shared__ int s_y0;                             // wave 1's draw, or kTailNotDrawn
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const Req rq = request(A, b);
  const int K = rq.k, V = A.V, R = A.R, nch = A.n_chunk;
  const int npl = (nch + 63) >> 6;
  const int nq = A.rows * npl;
  const int64_t rowg0 = (int64_t)b * A.rows;
  const uint32_t tag = A.tag;
  const int x = lane < K ? A.tokens[rq.x0 + lane] : -1;
  const bool valid = lane < K && (unsigned)x < (unsigned)V;
  const float T = A.temperature[b];
  const bool refused = !rq.ok || !(T > 0.f && T < __builtin_inff());
  // Every word the row pass writes for this request: the chunk partials of
  // its live rows, the uniforms of every position and the draft tokens'
  // logits. Wave 0 waits for all of them (also when the temperature refuses
  // the request); a ragged request with bad offsets has none.
  bool need[kFusedQ];
#pragma unroll
  for (int q = 0; q < kFusedQ; ++q) {
    const int rr = q < nq ? q / npl : 0, sc = (q < nq ? q % npl : 0) * 64 + lane;
    need[q] = rq.ok && q < nq && (rr < R ? rr <= K : rr - R < K) && sc < nch;
  }
  const bool need_u = rq.ok && lane < R;
  const bool need_g = rq.ok && valid;
  uint64_t* const us = A.tz_unif + 2 * ((int64_t)b * R + lane);
  // chunk sc of row rr: its word in run sc / cpw, and that run's max word
  const int cpw = A.cpw;
  auto word_of = [&](int q, bool max_word) {
    const int rr = q / npl, sc = (q % npl) * 64 + lane;
    const int w = sc / cpw;
    const int at = max_word ? min(cpw, nch - w * cpw) : sc - w * cpw;
    return run_words(A, rowg0 + rr, w) + at;
  };
  if (threadIdx.x == 0) { s_row0 = 0; s_seen = 0; s_y0 = kTailNotDrawn; }
  __syncthreads();
  auto flag_set = [](int* f, int v) { __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); };
  auto flag_get = [](int* f) { return __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); };

  bool got = false;
  float uacc = 0.f, usmp = 0.f, lx = kNegInf;
  uint64_t pm[kFusedQ], ps[kFusedQ];
  if (wave == 0) {
    uint64_t hx = 0ull, hu0 = 0ull, hu1 = 0ull;
#pragma unroll
    for (int q = 0; q < kFusedQ; ++q) { pm[q] = 0ull; ps[q] = 0ull; }
    got = !rq.ok;
    bool row0 = refused;                           // row 0 handed over (or never will be)
    if (refused && lane == 0) flag_set(&s_row0, 2);
    for (int spin = 0; rq.ok; ++spin) {
      bool miss = false, miss0 = false;
#pragma unroll
      for (int q = 0; q < kFusedQ; ++q) {
        if (need[q]) {
          if (!has_tag(pm[q], tag)) pm[q] = get_tag(word_of(q, true));
          if (!has_tag(ps[q], tag)) ps[q] = get_tag(word_of(q, false));
          const bool m = !(has_tag(pm[q], tag) && has_tag(ps[q], tag));
          miss |= m;
          if (q < npl) miss0 |= m;
        }
      }
      if (need_g && !has_tag(hx, tag)) hx = get_tag(A.tz_gath + rowg0 + lane);
      if (need_u) {
        if (!has_tag(hu0, tag)) hu0 = get_tag(us);
        if (!has_tag(hu1, tag)) hu1 = get_tag(us + 1);
      }
      const bool mg = need_g && !has_tag(hx, tag);
      const bool mu = need_u && !(has_tag(hu0, tag) && has_tag(hu1, tag));
      miss |= mg || mu;
      miss0 |= (lane == 0) && (mg || mu);
      if (!row0 && __ballot(miss0) == 0ull) {      // row 0 complete: hand it to wave 1
        row0 = true;
#pragma unroll
        for (int q = 0; q < kFusedQ; ++q)
          if (q < npl)                             // uniform
            s_p0[q * 64 + lane] = need[q] ? make_float2(tag_val(pm[q]), tag_val(ps[q]))
                                          : make_float2(kNegInf, 0.f);
        if (lane == 0) {
          s_u0 = tag_val(hu1);
          s_lx0 = need_g ? tag_val(hx) : kNegInf;
          flag_set(&s_row0, 1);
        }
      }
      if (__ballot(miss) == 0ull) { got = true; break; }
      if (spin >= A.spin_limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (!row0 && lane == 0) flag_set(&s_row0, 2);
    if (lane == 0) flag_set(&s_seen, got && rq.ok ? 1 : 2);
    if (!got) count_give_up(A);
    uacc = tag_val(hu0);
    usmp = tag_val(hu1);
    lx = need_g ? tag_val(hx) : kNegInf;
  } else if (wave == 1) {
    // the draw from row 0: the residual of a rejection at position 0, or the
    // bonus token when there are no drafts
    int st;
    while ((st = flag_get(&s_row0)) == 0) __builtin_amdgcn_s_sleep(1);
    if (st == 1) {
      const float c = kLog2e / T;
      float mi = kNegInf;
#pragma unroll
      for (int q = 0; q < kFusedQ; ++q)
        if (q < npl) mi = fmaxf(mi, s_p0[q * 64 + lane].x);
      mi = wave_max_all(mi);
      const int x0 = lane_i(x, 0);
      const float M = K > 0 ? fmaxf(mi, s_lx0 * c) : mi;
      const int xe = K > 0 ? x0 : -1;
      auto part_of = [&](int sc) { return s_p0[(sc >> 6) * 64 + (sc & 63)]; };
      int y = draw_from_partials<DT, kVec, kMask, false>(A, b, rq, 0, c, M, xe, s_u0, kNegInf, part_of);
      if (y < 0) y = ((unsigned)xe < (unsigned)V) ? xe : 0;    // residual without mass: p_0's mode
      if (lane == 0) s_y0 = y;
    }
  } else if (wave == 2) {
    // clear every tagged word for later calls once wave 0 has seen them all
    int st;
    while ((st = flag_get(&s_seen)) == 0) __builtin_amdgcn_s_sleep(1);
    if (st == 1) {
#pragma unroll
      for (int q = 0; q < kFusedQ; ++q) {
        if (need[q]) {
          clear_tag(word_of(q, true));
          clear_tag(word_of(q, false));
        }
      }
      if (need_g) clear_tag(A.tz_gath + rowg0 + lane);
      if (need_u) {
        clear_tag(us);
        clear_tag(us + 1);
      }
    }
  }
  if (wave == 0 && got && !refused && npl == 1) {
    // per-row (max, sum) with one partial per lane and row: every row's
    // reduction at once, independent chains the scheduler interleaves
    float mx[kFusedQ], sr[kFusedQ];
#pragma unroll
    for (int q = 0; q < kFusedQ; ++q) mx[q] = need[q] ? tag_val(pm[q]) : kNegInf;
#pragma unroll
    for (int q = 0; q < kFusedQ; ++q) mx[q] = q < A.rows ? wave_max_all(mx[q]) : kNegInf;
#pragma unroll
    for (int q = 0; q < kFusedQ; ++q) {
      const float mq = need[q] ? tag_val(pm[q]) : kNegInf;
      sr[q] = mq == kNegInf ? 0.f : tag_val(ps[q]) * fast_exp2(mq - mx[q]);
    }
#pragma unroll
    for (int q = 0; q < kFusedQ; ++q) sr[q] = q < A.rows ? wave_sum_all(sr[q]) : 0.f;
    if (lane < A.rows) {
      float m = kNegInf, sm = 0.f;
#pragma unroll
      for (int q = 0; q < kFusedQ; ++q) if (lane == q) { m = mx[q]; sm = sr[q]; }
      s_rowM[lane] = m;
      s_rowS[lane] = sm;
    }
  } else if (wave == 0 && got && !refused) {
    // per-row (max, sum): the row's largest chunk max, then the sum of the
    // chunk sums rescaled to it
    for (int rr = 0; rr < A.rows; ++rr) {          // uniform
      float m = kNegInf;
#pragma unroll
      for (int q = 0; q < kFusedQ; ++q)
        if (q >= rr * npl && q < (rr + 1) * npl && need[q]) m = fmaxf(m, tag_val(pm[q]));
      const float Mr = wave_max_all(m);
      float sr = 0.f;
#pragma unroll
      for (int q = 0; q < kFusedQ; ++q)
        if (q >= rr * npl && q < (rr + 1) * npl && need[q]) {
          const float mq = tag_val(pm[q]);
          sr += mq == kNegInf ? 0.f : tag_val(ps[q]) * fast_exp2(mq - Mr);
        }
      sr = wave_sum_all(sr);
      if (lane == 0) { s_rowM[rr] = Mr; s_rowS[rr] = sr; }
    }
  }
  __syncthreads();                                 // wave 1's draw is in s_y0
  if (wave != 0) return;
  int32_t* otok = A.out_tokens + (int64_t)b * A.out_cols;
  for (int j = K + 1 + lane; j < A.out_cols; j += 64) otok[j] = -1;   // columns past this request's drafts
  if (refused || !got) {
    if (lane <= K) otok[lane] = -1;
    if (lane < K && A.out_p) A.out_p[rq.x0 + lane] = 0.f;
    if (lane < K && A.out_q) A.out_q[rq.x0 + lane] = 0.f;
    if (lane == 0) A.out_len[b] = 0;
    return;
  }
  const float c = kLog2e / T;
  float p = 0.f, q = 0.f, Mx = kNegInf;
  if (lane < K) {
    // row `lane`'s sums leave x out: add its own term back for p(x)
    const float Mi = s_rowM[lane], Si = s_rowS[lane];
    Mx = fmaxf(Mi, lx * c);
    const float Sx = (Mi == kNegInf) ? 0.f : Si * fast_exp2(Mi - Mx);
    const float e = (valid && Mx != kNegInf) ? fast_exp2(fmaf(lx, c, -Mx)) : 0.f;
    const float St = Sx + e;
    p = St > 0.f ? e / St : 0.f;
    q = valid ? 1.f : 0.f;
    if (A.out_p) A.out_p[rq.x0 + lane] = p;
    if (A.out_q) A.out_q[rq.x0 + lane] = q;
  }
  const bool accept = uacc * q < p;
  const int rej = first_lane(lane < K && !accept);
  const int a = rej < 0 ? K : rej;
  if (lane <= K && lane != a) otok[lane] = lane < a ? x : -1;
  if (lane == 0) A.out_len[b] = a + 1;
  int y = a == 0 ? s_y0 : kTailNotDrawn;
  if (y == kTailNotDrawn) {                        // stopped past position 0: draw here
    const float ua = lane_f(usmp, a);
    const bool resid = a < K;
    const float M = resid ? lane_f(Mx, a) : s_rowM[a];
    const int xe = resid ? lane_i(x, a) : -1;
    // chunk s of row a sits in this lane's load a * npl + s / 64 (s = lane mod 64)
    auto part_of = [&](int sc) {
      const int qa = a * npl + (sc >> 6);          // uniform
      float2 v = make_float2(kNegInf, 0.f);
#pragma unroll
      for (int qq = 0; qq < kFusedQ; ++qq)
        if (qq == qa && need[qq]) v = make_float2(tag_val(pm[qq]), tag_val(ps[qq]));
      return v;
    };
    y = draw_from_partials<DT, kVec, kMask, false>(A, b, rq, a, c, M, xe, ua, kNegInf, part_of);
    if (y < 0) y = ((unsigned)xe < (unsigned)V) ? xe : 0;    // residual without mass: p_a's mode
  }
  if (lane == 0) otok[a] = y;
}

// kTagged: the partials come from the same launch's row pass (tagged slots).
template <bool kTagged>
__device__ void greedy_tail(const Args& A, int b, int* sg) {
  const int lane = threadIdx.x & 63;
  const Req rq = request(A, b);
  const int K = rq.k;
  const int x = lane < K ? A.tokens[rq.x0 + lane] : -1;
  WStaged ws;
  const float2 identity = make_float2(kNegInf, __int_as_float(INT_MAX));
  bool got = true;
  if constexpr (kTagged) {
    got = wstage_tagged(A, b, rq.ok ? K + 1 : 0, identity, ws);
    if (!got) count_give_up(A);
  } else {
    wstage_issue(A, b, A.rows, identity, ws);
  }
  merge_argmax_rows(A, b, A.rows, sg, ws);
  const int g = lane <= K ? sg[lane] : -1;
  const int mis = first_lane(lane < K && x != g);
  const int a = mis < 0 ? K : mis;
  int32_t* otok = A.out_tokens + (int64_t)b * A.out_cols;
  for (int j = K + 1 + lane; j < A.out_cols; j += 64) otok[j] = -1;   // columns past this request's drafts
  if (!rq.ok || !got) {                            // refused (ragged offsets; a wait that gave up)
    if (lane <= K) otok[lane] = -1;
    if (lane == 0) A.out_len[b] = 0;
    return;
  }
  if (lane <= K) {
    otok[lane] = lane < a ? x : (lane == a ? g : -1);
    if (A.out_aux) A.out_aux[rq.g0 + lane] = g;
  }
  if (lane == 0) A.out_len[b] = a + 1;
  if constexpr (kTagged) wclear_tagged(A, b, K + 1, ws);
}

// The tree's acceptance in parallel, one lane per node: a node is accepted
// when its token is its parent's argmax and its parent is accepted, settled
// one depth level at a time; the answer is the deepest accepted node (the
// lowest index among equals), and its root path is read off the parents.
template <bool kTagged>
__device__ void tree_tail(const Args& A, int b, int* sg) {
  const int lane = threadIdx.x & 63, N = A.n_nodes;
  const int xn = lane < N ? A.tokens[(int64_t)b * N + lane] : -1;
  // this request's tree: the call's static one, or its own row of a
  // dynamic batch (loaded with the tokens, checked below)
  int par = lane < N ? (A.dyn_parents ? A.dyn_parents[(int64_t)b * N + lane] : A.parent[lane]) : -1;
  int32_t* out = A.out_tokens + (int64_t)b * A.out_cols;
  auto refuse = [&]() {
    if (lane < N) out[lane] = -1;
    if (lane == 0) {
      A.out_len[b] = 0;
      if (A.out_aux) A.out_aux[b] = -1;
    }
  };
  WStaged ws;
  const float2 identity = make_float2(kNegInf, __int_as_float(INT_MAX));
  if constexpr (kTagged) {
    if (!wstage_tagged(A, b, N, identity, ws)) {   // the wait gave up: refuse the request
      count_give_up(A);
      refuse();
      return;
    }
  } else {
    wstage_issue(A, b, N, identity, ws);
  }
  int dep = lane < N ? A.depth[lane] : 0;
  if (A.dyn_parents) {
    // a row that is not a tree (the root's parent not -1, or a parent not
    // before its child) refuses its request; depths by N - 1 relaxation steps
    const bool bad = lane < N && (lane == 0 ? par != -1 : (par < 0 || par >= lane));
    if (__ballot(bad) != 0ull) {
      refuse();
      if constexpr (kTagged) wclear_tagged(A, b, N, ws);
      return;
    }
    dep = 0;
    for (int it = 1; it < N; ++it) {              // uniform; parents precede children
      const int pd = __shfl(dep, par < 0 ? 0 : par);
      dep = (lane > 0 && lane < N) ? pd + 1 : 0;
    }
  }
  merge_argmax_rows(A, b, N, sg, ws);
  const int g_par = sg[par < 0 ? 0 : par];
  const bool ok = lane == 0 || (lane < N && xn == g_par);
  const int max_depth = (int)wave_max_all((float)dep);
  int acc = lane == 0 ? 1 : 0;
  for (int d = 1; d <= max_depth; ++d) {           // uniform: all lanes take part
    const int pacc = __shfl(acc, par < 0 ? 0 : par);
    if (dep == d) acc = (ok && pacc) ? 1 : 0;
  }
  // deepest accepted node, lowest index among equals: key depth * 128 + 127 - node
  const int key = (lane < N && acc) ? dep * 128 + (127 - lane) : 0;
  const int kmax = (int)wave_max_all((float)key);
  const int best = 127 - (kmax & 127), len = kmax >> 7;
  uint64_t on_path = 0ull;
  for (int n = best; n > 0; n = __shfl(par, n)) on_path |= 1ull << n;   // uniform walk to the root
  // each position once: path nodes fill 0..len-1 (one node per depth), then
  // the argmax at the deepest node, then -1
  if (lane > 0 && lane < N && ((on_path >> lane) & 1ull)) out[dep - 1] = xn;
  if (lane == len) out[len] = sg[best];
  if (lane > len && lane < N) out[lane] = -1;
  if (lane == 0) {
    A.out_len[b] = len + 1;
    if (A.out_aux) A.out_aux[b] = best;
  }
  if constexpr (kTagged) wclear_tagged(A, b, N, ws);
}

// ------------------------------------------------- early-exit rounds ---
// The rule stops at the first rejection ("推测解码与 MTP" §2.1), so rows
// after it are never needed. Two rounds: position 0 alone, then positions
// 1..K together (each extra round costs a launch, a ticket and a chain of
// dependent loads, which measured more than the rows a finer split saves).
// A round reads the window's target rows (and draft rows) of the requests
// still open; the last workgroup of a
// request to finish its share then decides the window's positions in order
// with one wave: all accepted -> open for the next round; a rejection ->
// draw (or hand the residual to the residual pass) and close; position K ->
// bonus draw. Everything the decision reads
// from other workgroups (partials, the gathered logits, the uniforms) is
// published with agent-scope stores and fetched with agent-scope loads.

// (M, S) of rows r1 and (when r2 >= 0) r2 from their row-pass workgroup
// partials; the loads of both rows are issued before either merge.
__device__ void merge_rows(const Args& A, int b, int r1, int r2, float2* out1, float2* out2) {
  const int lane = threadIdx.x & 63;
  const float2* wp1 = A.wpart + ((int64_t)b * A.rows + r1) * A.wpr;
  const float2* wp2 = A.wpart + ((int64_t)b * A.rows + (r2 < 0 ? r1 : r2)) * A.wpr;
  float m1 = kNegInf, s1 = 0.f, m2 = kNegInf, s2 = 0.f;
  for (int w = lane; w < A.wpr; w += 64) {
    const float2 v1 = fetch(wp1 + w);
    const float2 v2 = r2 >= 0 ? fetch(wp2 + w) : make_float2(kNegInf, 0.f);
    ms_merge(m1, s1, v1.x, v1.y);
    ms_merge(m2, s2, v2.x, v2.y);
  }
  const float M1 = wave_max_all(m1);
  *out1 = make_float2(M1, wave_sum_all((m1 == kNegInf) ? 0.f : s1 * fast_exp2(m1 - M1)));
  if (r2 >= 0) {
    const float M2 = wave_max_all(m2);
    *out2 = make_float2(M2, wave_sum_all((m2 == kNegInf) ? 0.f : s2 * fast_exp2(m2 - M2)));
  }
}

// Position i of request b: accept (true: go on), or stop there (draw, or
// leave the residual to its pass) or, at i = K, draw the bonus token.
template <int MODE, int DT, bool kVec>
__device__ bool decide_position(const Args& A, int b, int i, float c, const Req& rq, int32_t* otok) {
  const int lane = threadIdx.x & 63;
  const int K = A.K, R = A.R, V = A.V;
  const int64_t rowg0 = (int64_t)b * A.rows;
  // every load the position needs, issued together: the draft token, the
  // gathered logits, the uniforms, the row's chunk partials for a draw (one
  // per lane when they fit) and the workgroup partials
  const int xt = i < K ? A.tokens[(int64_t)b * K + i] : -1;
  const float gx = i < K ? fetch(A.gath + rowg0 + i) : kNegInf;
  const float gd = (MODE == kExplicit && i < K) ? fetch(A.gath + rowg0 + R + i) : kNegInf;
  const float2 un = fetch(A.unif + (int64_t)b * R + i);
  const float2* part_i = A.part + (rowg0 + i) * A.n_chunk;
  const bool pre_on = A.n_chunk <= 64 && (MODE == kOneHot || i == K);
  const float2 pre = (pre_on && lane < A.n_chunk) ? fetch(part_i + lane) : make_float2(kNegInf, 0.f);
  auto part_of = [&](int s) { return pre_on ? pre : fetch(part_i + s); };   // s == lane when pre_on
  float2 mp, mq = make_float2(kNegInf, 0.f);
  merge_rows(A, b, i, (MODE == kExplicit && i < K) ? R + i : -1, &mp, &mq);
  int y;
  if (i < K) {
    const int x = xt;
    const bool valid = (unsigned)x < (unsigned)V;
    const float lx = valid ? gx : kNegInf;
    float p, q, Mx = mp.x;
    bool accept;
    if (MODE == kOneHot) {
      // the row's sums leave x out: add its own term back for p(x)
      Mx = fmaxf(mp.x, lx * c);
      const float Sx = (mp.x == kNegInf) ? 0.f : mp.y * fast_exp2(mp.x - Mx);
      const float e = (valid && Mx != kNegInf) ? fast_exp2(fmaf(lx, c, -Mx)) : 0.f;
      const float St = Sx + e;
      p = St > 0.f ? e / St : 0.f;
      q = valid ? 1.f : 0.f;
      accept = un.x * q < p;
    } else {
      const float ld = valid ? gd : kNegInf;
      const float dp = fmaf(lx, c, -mp.x), dq = fmaf(ld, c, -mq.x);
      p = (valid && mp.y > 0.f) ? fast_exp2(dp) / mp.y : 0.f;
      q = (valid && mq.y > 0.f) ? fast_exp2(dq) / mq.y : 0.f;
      const float lp = (valid && mp.y > 0.f) ? dp - __log2f(mp.y) : kNegInf;
      const float lq = (valid && mq.y > 0.f) ? dq - __log2f(mq.y) : kNegInf;
      accept = __log2f(un.x) + lq < lp;
      if (!accept && lane == 0) {                  // the residual pass draws this one
        Record rc;
        rc.a = i; rc.pending = 1; rc.c = c; rc.u = un.y;
        rc.Mp = mp.x; rc.Sp = mp.y; rc.Mq = mq.x; rc.Sq = mq.y;
        A.rec[b] = rc;
      }
    }
    if (lane == 0) {
      if (A.out_p) A.out_p[(int64_t)b * K + i] = p;
      if (A.out_q) A.out_q[(int64_t)b * K + i] = q;
    }
    if (accept) {
      if (lane == 0) otok[i] = x;
      return true;
    }
    // stop at a = i: positions after it are padding, their p and q not reported
    if (lane > i && lane <= K) otok[lane] = -1;
    if (lane > i && lane < K) {
      if (A.out_p) A.out_p[(int64_t)b * K + lane] = 0.f;
      if (A.out_q) A.out_q[(int64_t)b * K + lane] = 0.f;
    }
    if (lane == 0) {
      A.out_len[b] = i + 1;
      A.alive[b] = 0;
    }
    if (MODE == kExplicit) return false;
    y = draw_from_partials<DT, kVec, false, false>(A, b, rq, i, c, Mx, x, un.y, kNegInf, part_of);
    if (y < 0) y = valid ? x : 0;                  // residual without mass: p's mode
  } else {                                         // all K accepted: the bonus token from p_K
    y = draw_from_partials<DT, kVec, false, false>(A, b, rq, K, c, mp.x, -1, un.y, kNegInf, part_of);
    if (y < 0) y = 0;
    if (lane == 0) {
      A.out_len[b] = K + 1;
      A.alive[b] = 0;
      if (MODE == kExplicit) A.rec[b].pending = 0;
    }
  }
  if (lane == 0) otok[i] = y;
  return false;
}

// The positions round..round_hi of request b, in order, until one stops it.
template <int MODE, int DT, bool kVec>
__device__ void round_decide(const Args& A, int b) {
  const int lane = threadIdx.x & 63;
  const int K = A.K;
  const Req rq = request(A, b);
  int32_t* otok = A.out_tokens + (int64_t)b * A.out_cols;
  const float T = A.temperature[b];
  if (!(T > 0.f && T < __builtin_inff())) {        // refused request (round 0 only)
    if (lane <= K) otok[lane] = -1;
    if (lane < K && A.out_p) A.out_p[(int64_t)b * K + lane] = 0.f;
    if (lane < K && A.out_q) A.out_q[(int64_t)b * K + lane] = 0.f;
    if (lane == 0) {
      A.out_len[b] = 0;
      A.alive[b] = 0;
      if (MODE == kExplicit) A.rec[b].pending = 0;
    }
    return;
  }
  const float c = kLog2e / T;
  for (int i = A.round; i <= A.round_hi; ++i)
    if (!decide_position<MODE, DT, kVec>(A, b, i, c, rq, otok)) return;
  if (lane == 0) A.alive[b] = 1;                   // every position of the window accepted
}

// ------------------------------------------------------------ row pass ---
// Logit (j, k) of a lane's chunk: word k / kPerWord of vector j, widened.
template <int DT>
__device__ __forceinline__ uint32_t& raw_word(ChunkRaw& r, int j, int w) {
  return w == 0 ? r.v[j].x : w == 1 ? r.v[j].y : w == 2 ? r.v[j].z : r.v[j].w;
}
template <int DT>
__device__ __forceinline__ float raw_elem(ChunkRaw& r, int j, int k) {
  if constexpr (DT == kF32) {
    return __uint_as_float(raw_word<DT>(r, j, k));
  } else {
    const uint32_t w = raw_word<DT>(r, j, k >> 1);
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
  }
}
// Sets logit (j, k) to -inf when `hit`.
template <int DT>
__device__ __forceinline__ void raw_mask(ChunkRaw& r, int j, int k, bool hit) {
  if constexpr (DT == kF32) {
    uint32_t& w = raw_word<DT>(r, j, k);
    w = hit ? 0xFF800000u : w;
  } else {
    uint32_t& w = raw_word<DT>(r, j, k >> 1);
    const uint32_t masked = (k & 1) ? ((w & 0x0000FFFFu) | 0xFF800000u) : ((w & 0xFFFF0000u) | 0xFF80u);
    w = hit ? masked : w;
  }
}
// Opaque to the optimiser: the second pass over a chunk re-widens the
// packed words instead of keeping every widened logit live across passes.
__device__ __forceinline__ void touch(ChunkRaw& r) {
#pragma unroll
  for (int j = 0; j < kLoadsPerLane; ++j)
    asm volatile("" : "+v"(r.v[j].x), "+v"(r.v[j].y), "+v"(r.v[j].z), "+v"(r.v[j].w));
}

// Running softmax reference of one wave over the chunks it streams. Each
// lane sums 2^(y - ref) against its own reference `ref` (a scaled logit
// the lane has seen, so y - ref only exceeds 64 for data that triggers a
// recount); the wave's partial is taken against M, the largest lane
// reference, with f = 2^(ref - M) cached until some lane's reference moves.
struct RefState {
  float ref = kNegInf;   // lane
  float f = 0.f;         // lane: 2^(ref - M), 0 while ref is -inf
  float M = kNegInf;     // wave-uniform
  bool first = true;     // wave-uniform: no chunk seen yet
};

// One chunk's partial from one wave (after the grammar bitmask, if any, has
// turned disallowed logits into -inf): (M, sum 2^(y - M)) for sampling, where
// M is a reference no larger than the row's maximum scaled logit (and, for
// a chunk with finite logits, no smaller than any of them minus 64);
// (max logit, lowest index of it) for greedy/tree. With a draft token xe in
// this chunk, its logit goes to `gath` and, for one-hot drafts, it is left
// out of the sums (kPub: stored with an agent-scope store, for readers in
// the same launch). `r` holds the lane's four 16-byte vectors.
template <int MODE, int DT, bool kMask, bool kPub>
__device__ __forceinline__ float2 chunk_partial(ChunkRaw& r, const MaskRaw& mk, int c0, int xe, float c,
                                                float* gath, RefState& st) {
  constexpr int kPer = Elem<DT>::kPerVec;
  const int lane0 = (threadIdx.x & 63) * kPer;   // first logit of the lane's vector 0
  if constexpr (kMask) apply_mask<DT>(r, mk);     // disallowed logits read as -inf from here on
  if constexpr (MODE == kOneHot || MODE == kExplicit) {
    const int dx = xe - c0;                       // the draft token's offset in this chunk
    if (xe >= 0 && (unsigned)dx < (unsigned)Chunk<DT>::kElems) {
      // only the wave holding the chunk with the token gets here (uniform
      // branch). Vector, lane and 32-bit word of the token are uniform.
      constexpr int kWordElems = kPer / 4;        // logits per 32-bit word
      const int vec = dx / kPer;
      const int jt = vec >> 6, lt = vec & 63;
      const int wt = (dx % kPer) / kWordElems, half = (dx % kPer) % kWordElems;
      const bool own = (threadIdx.x & 63) == lt;
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < kLoadsPerLane; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) w = (j == jt && q == wt) ? raw_word<DT>(r, j, q) : w;
      if (own) {
        float lx;
        if constexpr (DT == kF32) lx = __uint_as_float(w);
        else lx = half ? bf16_hi(w) : bf16_lo(w);
        if constexpr (kPub) publish(gath, lx);    // once per row
        else *gath = lx;
      }
      if (MODE == kOneHot) {
        uint32_t masked;
        if constexpr (DT == kF32) masked = 0xFF800000u;
        else masked = half ? ((w & 0x0000FFFFu) | 0xFF800000u) : ((w & 0xFFFF0000u) | 0xFF80u);
#pragma unroll
        for (int j = 0; j < kLoadsPerLane; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t& dst = raw_word<DT>(r, j, q);
            dst = (own && j == jt && q == wt) ? masked : dst;
          }
      }
    }
    touch(r);
    const bool seeded = st.first;                 // uniform: the references move
    if (seeded) {
      // seed each lane's reference with the largest logit of its first vector
      float m0 = kNegInf;
#pragma unroll
      for (int k = 0; k < kPer; ++k) m0 = fmaxf(m0, raw_elem<DT>(r, 0, k));
      st.ref = m0 * c;                            // -inf stays -inf
      st.first = false;
    }
    // One pass: sum 2^(y - ref). A lane with no finite reference yet gets
    // NaN or inf here, and one with a logit more than 64 above its
    // reference gets a sum above 2^64: both recount exactly below.
    float acc[kLoadsPerLane];
#pragma unroll
    for (int j = 0; j < kLoadsPerLane; ++j) {
      acc[j] = 0.f;
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc[j] += fast_exp2(fmaf(raw_elem<DT>(r, j, k), c, -st.ref));
    }
    float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const bool recount = !(s <= 0x1p64f);
    if (seeded || __ballot(recount) != 0ull) {    // uniform branch, rare after the first chunk
      if (recount) {
        touch(r);                                 // reconvert rather than keep 32 values live
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < kLoadsPerLane; ++j)
#pragma unroll
          for (int k = 0; k < kPer; ++k) mx = fmaxf(mx, raw_elem<DT>(r, j, k));
        st.ref = fmaxf(st.ref, mx * c);
        touch(r);
        s = 0.f;
        if (st.ref != kNegInf) {
#pragma unroll
          for (int j = 0; j < kLoadsPerLane; ++j) {
            acc[j] = 0.f;
#pragma unroll
            for (int k = 0; k < kPer; ++k) acc[j] += fast_exp2(fmaf(raw_elem<DT>(r, j, k), c, -st.ref));
          }
          s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
      }
      st.M = wave_max_all(st.ref);
      st.f = (st.ref == kNegInf) ? 0.f : fast_exp2(st.ref - st.M);
    }
    s = wave_sum_all(s * st.f);
    return make_float2(st.M, s);
  } else {
    float best = raw_elem<DT>(r, 0, 0);
    int bi = c0 + lane0;
#pragma unroll
    for (int j = 0; j < kLoadsPerLane; ++j) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const float v = raw_elem<DT>(r, j, k);
        if (v > best) { best = v; bi = c0 + lane0 + j * 64 * kPer + k; }
      }
    }
    wave_argmax_all(best, bi);
    return make_float2(best, __int_as_float(bi));
  }
}

// Workgroup w owns chunks [c_lo, c_hi) of row (w / wpr); wave v of it
// streams chunks c_lo + v, c_lo + v + 4, ... Full chunks go through a
// two-deep pipeline of raw 16-byte loads; a row's last, partial chunk and
// rows that are not 16-byte aligned take the checked element path.
// kRound: one early-exit round (rows round..round_hi of the open requests),
// the decision taken at the end by the request's last workgroup.
// kFused: a one-launch call; the B workgroups after the row pass's run the
// rule, one request each, on the row pass's tagged results.
template <int MODE, int DT, bool kVec, bool kMask, bool kRound, bool kFused>
__global__ __launch_bounds__(kThreads) void sv_rows_kernel(Args A) {
  constexpr int kCE = Chunk<DT>::kElems;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  if constexpr (kFused) {
    if (blockIdx.x >= (unsigned)A.n_rowwg) {      // a tail workgroup
      const int bt = (int)(blockIdx.x - (unsigned)A.n_rowwg);
      if constexpr (MODE == kOneHot) {
        fused_sample_tail<DT, kVec, kMask>(A, bt);   // every wave takes part
      } else if constexpr (MODE == kExplicit) {
        static_assert(MODE != kExplicit, "calls with draft logits never take one launch");
      } else if (wave == 0) {                     // one wave does the work
        __shared__ int s_g[SV_MAX_TREE_NODES];
        if constexpr (MODE == kGreedy) greedy_tail<true>(A, bt, s_g);
        else tree_tail<true>(A, bt, s_g);
      }
      return;
    }
  }
  const int wi = (int)(blockIdx.x % (unsigned)A.wpr);
  const int slot = (int)(blockIdx.x / (unsigned)A.wpr);
  int b, r;
  if constexpr (!kRound) {                        // every row of every request
    b = slot / A.rows;
    r = slot % A.rows;
  } else {                                        // target (and draft) rows round..round_hi
    b = slot / A.round_rows;
    const int j = slot % A.round_rows, w = A.round_hi - A.round + 1;
    r = j < w ? A.round + j : A.R + A.round + (j - w);
    if (A.round > 0 && !A.alive[b]) return;       // the request stopped in an earlier round
  }
  const int rowg = b * A.rows + r;
  const Req rq = request(A, b);
  if (A.cu && !row_live(A, rq, r)) return;        // a ragged request's padding rows: no work
  const char* row = row_ptr(A, rq, r);
  const uint32_t* mrow = kMask ? mask_row(A, b, r < A.R ? r : r - A.R) : nullptr;
  const int c_lo = wi * A.cpw;
  const int c_hi = min(c_lo + A.cpw, A.n_chunk);
  // Partials collect in LDS and leave in one store at the end: no global
  // store sits between the chunk loads.
  __shared__ float2 s_part[kMaxChunksPerWg];
  __shared__ float2 s_unif[SV_MAX_DRAFT + 1];
  __shared__ float s_gx;                          // one-launch calls: the draft token's logit
  float* gath = kFused ? &s_gx : A.gath + rowg;

  int ch = c_lo + wave;
  const int ch_end = kVec ? min(c_hi, A.n_full) : c_lo;
  RefState rs;
  const bool piped = ch < ch_end;
  ChunkRaw ra, rb;
  MaskRaw ma, mb;
  if (piped) {                                     // first loads before anything else
    issue_chunk<DT>(row, (int64_t)ch * kCE, ra);
    if (kMask) issue_mask<DT>(mrow, (int64_t)ch * kCE, A.mask_words, ma);
  }
  __builtin_amdgcn_sched_barrier(0);

  // The draft token of this row (if any): its logit is kept for the tail,
  // and with one-hot drafts it is left out of the row's sums.
  int xe = -1;
  float c = 0.f;
  if (MODE == kOneHot || MODE == kExplicit) {
    const int i = r < A.R ? r : r - A.R;
    if (i < rq.k) xe = A.tokens[rq.x0 + i];
    c = kLog2e / A.temperature[b];
    // The two uniforms of every position i <= K of request b, one lane per
    // position: drawn by one wave of the last (shortest) workgroup of the
    // request's first row while its first loads are in flight, and left for
    // the tail, which would otherwise wait on this chain of 64-bit multiplies.
    if (r == 0 && wi == A.wpr - 1 && wave == 0 && lane < A.R) {
      const Philox4 rnd = philox4x64_10((uint64_t)lane, (uint64_t)b, A.offset, 0ull, A.seeds[b], 0ull);
      s_unif[lane] = make_float2(top24(rnd.w0), top24(rnd.w1));
    }
  }

  if (piped) {
    // The prefetch is unconditional so that every iteration has the same
    // loads in flight (the waits stay exact); past the end it re-reads the
    // current chunk, which the L2 still holds.
    while (true) {
      int nx = ch + kWaves;
      bool more = nx < ch_end;
      issue_chunk<DT>(row, (int64_t)(more ? nx : ch) * kCE, rb);
      if (kMask) issue_mask<DT>(mrow, (int64_t)(more ? nx : ch) * kCE, A.mask_words, mb);
      __builtin_amdgcn_sched_barrier(0);           // keep the prefetch ahead of the math
      {
        const float2 res = chunk_partial<MODE, DT, kMask, kRound>(ra, ma, ch * kCE, xe, c, gath, rs);
        if (lane == 0) s_part[ch - c_lo] = res;
      }
      ch = nx;
      if (!more) break;
      nx = ch + kWaves;
      more = nx < ch_end;
      issue_chunk<DT>(row, (int64_t)(more ? nx : ch) * kCE, ra);
      if (kMask) issue_mask<DT>(mrow, (int64_t)(more ? nx : ch) * kCE, A.mask_words, ma);
      __builtin_amdgcn_sched_barrier(0);
      {
        const float2 res = chunk_partial<MODE, DT, kMask, kRound>(rb, mb, ch * kCE, xe, c, gath, rs);
        if (lane == 0) s_part[ch - c_lo] = res;
      }
      ch = nx;
      if (!more) break;
    }
  }
  for (; ch < c_hi; ch += kWaves) {               // checked path
    ChunkRaw rr;
    MaskRaw mr;
    load_chunk_checked<DT, kVec>(row, (int64_t)ch * kCE, A.V, rr);
    if (kMask) issue_mask<DT>(mrow, (int64_t)ch * kCE, A.mask_words, mr);
    const float2 res = chunk_partial<MODE, DT, kMask, kRound>(rr, mr, ch * kCE, xe, c, gath, rs);
    if (lane == 0) s_part[ch - c_lo] = res;
  }
  __syncthreads();
  if constexpr (kFused) {
    // one-launch call: tagged stores for the tail workgroups, then done
    // (nothing waits for them). Sampling: every chunk partial, the draft
    // token's logit (by the workgroup whose run holds it) and the uniforms;
    // greedy / tree: the workgroup's argmax.
    const uint32_t tag = A.tag;
    if (b == A.drop_req) return;                  // test hook: this request's tail must give up
    if constexpr (MODE == kOneHot || MODE == kExplicit) {
      // one word per chunk, its sum rescaled to the run's largest chunk max,
      // then that max: n + 1 words from one store instruction (a wave's
      // stores hold its slot until they are acknowledged, so they are few)
      if (wave == 0) {
        const int n = c_hi - c_lo;
        float m = kNegInf;
        for (int i = lane; i < n; i += 64) m = fmaxf(m, s_part[i].x);
        const float mw = wave_max_all(m);
        uint64_t* tp = run_words(A, rowg, wi);
        for (int i = lane; i <= n; i += 64) {
          float v = mw;
          if (i < n) v = s_part[i].x == kNegInf ? 0.f : s_part[i].y * fast_exp2(s_part[i].x - mw);
          put_tag(tp + i, v, tag);
        }
      }
      if (tid == 0 && (unsigned)xe < (unsigned)A.V && xe / kCE >= c_lo && xe / kCE < c_hi)
        put_tag(A.tz_gath + rowg, s_gx, tag);
      if (r == 0 && wi == A.wpr - 1 && tid < A.R) {
        uint64_t* tu = A.tz_unif + 2 * ((int64_t)b * A.R + tid);
        put_tag(tu, s_unif[tid].x, tag);
        put_tag(tu + 1, s_unif[tid].y, tag);
      }
    } else if (wave == 0) {
      float v = kNegInf;
      int idx = INT_MAX;
      for (int i = lane; i < c_hi - c_lo; i += 64) am_step(v, idx, s_part[i].x, __float_as_int(s_part[i].y));
      wave_argmax_all(v, idx);
      if (lane == 0) {
        uint64_t* tw = A.tz_part + 2 * ((int64_t)rowg * A.wpr + wi);
        put_tag(tw, v, tag);
        put_tag(tw + 1, __int_as_float(idx), tag);
      }
    }
    return;
  }
  float2* part = A.part + (int64_t)rowg * A.n_chunk;
  for (int i = tid; i < c_hi - c_lo; i += kThreads) {
    if constexpr (kRound) publish(part + c_lo + i, s_part[i]);
    else part[c_lo + i] = s_part[i];
  }
  if (MODE == kOneHot || MODE == kExplicit) {
    if (r == 0 && wi == A.wpr - 1 && tid < A.R) {
      if constexpr (kRound) publish(A.unif + (int64_t)b * A.R + tid, s_unif[tid]);
      else A.unif[(int64_t)b * A.R + tid] = s_unif[tid];
    }
  }
  // wave 0 also folds the workgroup's partials into one, so the tail merges
  // wpr values per row instead of n_chunk
  if (wave == 0) {
    float2 acc;
    if constexpr (MODE == kOneHot || MODE == kExplicit) {
      float m = kNegInf, s = 0.f;
      for (int i = lane; i < c_hi - c_lo; i += 64) ms_merge(m, s, s_part[i].x, s_part[i].y);
      const float wm = wave_max_all(m);
      s = wave_sum_all((m == kNegInf) ? 0.f : s * fast_exp2(m - wm));
      acc = make_float2(wm, s);
    } else {
      float v = kNegInf;
      int idx = INT_MAX;
      for (int i = lane; i < c_hi - c_lo; i += 64) am_step(v, idx, s_part[i].x, __float_as_int(s_part[i].y));
      wave_argmax_all(v, idx);
      acc = make_float2(v, __int_as_float(idx));
    }
    if (lane == 0) {
      if constexpr (kRound) publish(A.wpart + (int64_t)rowg * A.wpr + wi, acc);
      else A.wpart[(int64_t)rowg * A.wpr + wi] = acc;
    }
  }
  if constexpr (kRound && (MODE == kOneHot || MODE == kExplicit)) {
    __shared__ int s_last;
    if (!last_of_request(A.counters + b, (unsigned)(A.round_rows * A.wpr), &s_last)) return;
    if (wave == 0) round_decide<MODE, DT, kVec>(A, b);
  }
}

// One wave per request: the rule on the merged partials. The launch
// boundary after the row pass is the only synchronisation the tail needs.
template <int MODE, int DT, bool kVec, bool kMask>
__global__ __launch_bounds__(64) void sv_tail_kernel(Args A) {
  __shared__ TailLds S;
  const int b = blockIdx.x;
  if constexpr (MODE == kOneHot || MODE == kExplicit) {
    sample_tail<DT, kVec, MODE, kMask>(A, b, S);
  } else if constexpr (MODE == kGreedy) {
    greedy_tail<false>(A, b, S.g);
  } else {
    tree_tail<false>(A, b, S.g);
  }
}

// ------------------------------------------------- top-k / top-p filters ---
// The sampler's filters, applied to p and, with draft logits, to q (the
// sampling parameters used with speculation in "Speculative Decoding
// Guide", vLLM-Ascend): top-k keeps the logits at least the k-th largest;
// top-p then keeps the largest cut whose upper set holds top_p of the
// remaining mass; ties at a cut are kept. One workgroup per row finds each
// cut as a logit value by descent over histograms of the log2 weight
//   D = l * log2(e) / T - Mref   (fp64; Mref = the row's largest l * log2(e) / T)
// in 1024 buckets of width 1/16 over [0, 64), refined 256-fold per level
// (at most three levels) until the bucket holding the cut has at most
// kSelCap logits. Those are cut exactly: the mass of each one's upper set
// among them (rank_cut), or a sort and a scan. A cut more than 64 below
// the largest log2 weight keeps the whole row (the weights it would drop
// are below 2^-64 of the largest).

constexpr int kSelBuckets0 = 1024;                // first level: width 1/16 over [0, 64)
constexpr int kSelBuckets = 256;                  // refinement levels
constexpr int kSelCap = 2048;
constexpr int kSelLevels = 3;

// bf16 rows: the one-pass search's table (see hist_pass).
constexpr int kHBins = 4096;                      // per sign: magnitudes [2^-16, 2^16)
constexpr uint32_t kHMagLo = 0x3780u;             // bf16 magnitude bits of 2^-16
constexpr int kHOrd = 2 * kHBins + 2;             // ordered positions (hist_value)
// Word of magnitude m (table: kHMagLo <= m < kHMagLo + kHBins) and sign s:
// kHOff + (m - kHMagLo) + s * kHNeg, the negative table right after the
// positive one (the sign bit, shifted, is the byte offset of the negative
// table). Values outside the table are counted at their sign's last word
// and taken out again after the pass.
constexpr int kHOff = 0, kHNeg = kHBins;
constexpr int kHWords = 2 * kHBins;
static_assert(kHNeg * 4 == 0x4000, "the sign bit shifted right by one is the negative table's byte offset");

struct alignas(16) SelLds {
  union {
    struct {
      unsigned cnt[kSelBuckets0];
      double mass[kSelBuckets0];
      uint32_t key[kSelCap];
      double w[kSelCap];
    };
    uint32_t hcnt[kHWords];                        // the positive table, then the negative one
  };
  double scan[kThreads];
  double tab[64];                                  // 2^(j / 64)
  double wtot[kWaves], wtot2[kWaves];             // wave totals of the count and mass scans
  float wsum[kWaves];
  float tiny_w[kWaves][3];                         // per wave: sums of tiny l, l^2, l^3
  int n, sel;
  uint32_t kfloor;
  unsigned tiny_n, ninf_n, tiny_max;               // tiny count, -inf count, largest tiny order key
  int big;                                         // a value outside the table that is not -inf
  int sel_max[kWaves], sel_k[kWaves], sel_p[kWaves];   // each wave's smallest pick candidate
  uint32_t kcut, kmin;                             // rank_cut's picks
};

// Total order of logit values as unsigned keys (-0 sorts with +0).
__device__ __forceinline__ uint32_t order_key(float l) {
  uint32_t u = __float_as_uint(l);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// 2^D in fp64 (relative error ~1e-15): 2^n * 2^(j/64) (table) * e^r with
// r = (f - j/64) ln 2 in [0, ln2/64) by its Taylor series to r^5.
__device__ __forceinline__ double exp2_weight(double D, const double* tab) {
  if (!(D > -1000.0)) return 0.0;
  const double n = floor(D), f = D - n;
  const int j = min((int)(f * 64.0), 63);
  const double r = (f - j * (1.0 / 64.0)) * 0.69314718055994530942;
  double e = 1.0 / 120.0;
  e = fma(e, r, 1.0 / 24.0);
  e = fma(e, r, 1.0 / 6.0);
  e = fma(e, r, 0.5);
  e = fma(e, r, 1.0);
  e = fma(e, r, 1.0);
  return ldexp(tab[j] * e, (int)n);
}

// Bucket of a logit at `level` inside bucket `parent` (its global index at
// level - 1), or -1 outside it. Non-increasing in the logit.
__device__ __forceinline__ int sel_bucket(double D, int level, int64_t parent) {
  if (level == 0) {
    const double t = -16.0 * D;
    if (!(t < (double)(kSelBuckets0 - 1))) return kSelBuckets0 - 1;   // also -inf and NaN
    return t > 0.0 ? (int)t : 0;
  }
  const double scale = level == 1 ? 4096.0 : 1048576.0;
  const double lo = (double)parent * kSelBuckets;
  const double t = fmax(-D, 0.0) * scale;
  if (!(t >= lo && t < lo + kSelBuckets)) return -1;
  return (int)(t - lo);
}

// Inclusive scan of one double per thread over a workgroup of NT threads
// (lanes in order within a wave, then waves in order). *excl gets the
// previous thread's result bit for bit (0 for thread 0) and *total the
// workgroup's sum, so that exactly the thread whose range holds a crossing
// of a threshold sees excl < t <= incl (up to the order of equal partial
// sums). wtot: NT / 64 doubles; kFree: no thread reads them at the call
// (else a barrier comes first).
template <int kCtrl, int kRows = 0xF>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, kRows, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, kRows, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Lane l's value of v, in every lane (l wave-uniform).
__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive scan over the wave's lanes: shifts within rows of 16 lanes,
// then the broadcasts of row ends (lanes without a source add 0).
__device__ __forceinline__ double wave_scan_incl_d(double v) {
  v += dpp_d<0x111>(v);
  v += dpp_d<0x112>(v);
  v += dpp_d<0x114>(v);
  v += dpp_d<0x118>(v);
  v += dpp_d<0x142, 0xA>(v);
  v += dpp_d<0x143, 0xC>(v);
  return v;
}

template <int NT, bool kFree = false>
__device__ __forceinline__ double wg_scan(double v, double* wtot, double* excl, double* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_incl_d(v);
  if (!kFree) __syncthreads();                     // earlier readers of wtot are done
  if (lane == 63) wtot[wave] = v;
  __syncthreads();
  double pre = 0.0, tot = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w == wave) pre = tot;
    tot += wtot[w];
  }
  const double incl = pre + v;
  const double prev = __shfl_up(incl, 1);
  *excl = lane == 0 ? pre : prev;
  *total = tot;
  return incl;
}

// Every logit of a row once (f(l, index)), chunk by chunk, the next chunk's
// load in flight during the current chunk's math; past the row's end f
// sees -inf. Always inlined: called out of line, a lambda's captured
// references put its state in scratch memory (the bf16 select kernel's
// fallback path gave that kernel a private segment).
template <int DT, bool kVec, class F>
__device__ __forceinline__ void for_each_logit(const char* row, int n_chunk, int V, F f) {
  constexpr int kCE = Chunk<DT>::kElems, kPT = Chunk<DT>::kPerThread;
  float nx[kPT];
  auto load = [&](int ch) {
    if (ch < n_chunk) {
      load_chunk_wg<DT, kVec>(row, (int64_t)ch * kCE, V, nx);
    } else {
#pragma unroll
      for (int k = 0; k < kPT; ++k) nx[k] = kNegInf;
    }
  };
  load(0);
  for (int ch = 0; ch < n_chunk; ++ch) {
    float x[kPT];
#pragma unroll
    for (int k = 0; k < kPT; ++k) x[k] = nx[k];
    if (ch + 1 < n_chunk) load(ch + 1);
    // padding past the row reads as -inf: a weight of zero in the last bucket
#pragma unroll
    for (int k = 0; k < kPT; ++k) f(x[k], (int64_t)ch * kCE + (int64_t)threadIdx.x * kPT + k);
  }
}

// The cut search's two views of a row. StreamRow reads it from memory
// with a workgroup of kThreads (for_each_logit); LdsRow is a row that a
// workgroup of NT threads has copied to LDS as 16-byte vectors, -inf past
// the row's end. each(f) calls f(l, index) once for every logit of the row
// (and the padding of its last vector).
template <int DT, bool kVec>
struct StreamRow {
  static constexpr int kNT = kThreads;
  const char* row;
  int n_chunk, V;
  template <class F>
  __device__ __forceinline__ void each(F f) const { for_each_logit<DT, kVec>(row, n_chunk, V, f); }
};

template <int NT, int NV>
struct LdsRow {
  static constexpr int kNT = NT;
  const float4* vec;
  int n_vec;                                       // at most NV * NT
  template <class F>
  __device__ __forceinline__ void each(F f) const {
    float4 q[NV];                                  // every read of the pass in flight at once
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = j * NT + threadIdx.x;
      q[j] = v < n_vec ? vec[v] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t e = (int64_t)(j * NT + threadIdx.x) * 4;
      f(q[j].x, e);
      f(q[j].y, e + 1);
      f(q[j].z, e + 2);
      f(q[j].w, e + 3);
    }
  }
};

// Descending bitonic sort of the first n collected entries (padded to a
// power of two with key 0, below every logit's key), by the NT threads of
// the workgroup.
template <int NT, class LT>
__device__ void sort_collected(LT& L, int n) {
  int np = 2;
  while (np < n) np <<= 1;
  for (int i = n + threadIdx.x; i < np; i += NT) {
    L.key[i] = 0u;
    L.w[i] = 0.0;
  }
  __syncthreads();
  for (int size = 2; size <= np; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (np >> 1); i += NT) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint32_t a = L.key[lo], c = L.key[hi];
        if (desc ? (a < c) : (a > c)) {
          L.key[lo] = c;
          L.key[hi] = a;
          const double t = L.w[lo];
          L.w[lo] = L.w[hi];
          L.w[hi] = t;
        }
      }
      __syncthreads();
    }
}

// Sorts the n collected logits (key, weight) by value, largest first, and
// returns the key at which above + their running sum first reaches target
// (falling short keeps them all: rounding at the row's end).
template <int NT, class LT>
__device__ uint32_t scan_collected(LT& L, int n, double above, double target) {
  const int tid = threadIdx.x;
  sort_collected<NT>(L, n);
  constexpr int kPer = kSelCap / NT;
  double loc = 0.0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid * kPer + j;
    loc += e < n ? L.w[e] : 0.0;
  }
  double excl, all;
  wg_scan<NT>(loc, L.wtot, &excl, &all);
  if (tid == 0) L.sel = INT_MAX;
  __syncthreads();
  double run = above + excl;
  for (int j = 0; j < kPer; ++j) {
    const int e = tid * kPer + j;
    if (e >= n) break;
    run += L.w[e];
    if (run >= target) {
      atomicMin(&L.sel, e);
      break;
    }
  }
  __syncthreads();
  const int sel = L.sel;
  uint32_t k = 0u;
  if (sel != INT_MAX) k = L.key[sel];
  else if (n > 0) k = L.key[n - 1];               // short of the target: the whole set
  __syncthreads();
  return k;
}

// The same cut as scan_collected for n <= NT collected logits, without the
// sort: the mass of the upper set {l >= l_i} of each logit i, and the cut
// is the largest key whose upper set brings above to target (falling
// short: as scan_collected). With n <= NT / 4, four neighbouring threads
// share logit i, each summing a quarter of the entries (combined in the
// quad); else one thread per logit. L.kcut must hold 0 and L.kmin the
// smallest collected key, both set before the barrier that ends the
// collection.
template <int NT, class LT>
__device__ uint32_t rank_cut(LT& L, int n, double above, double target) {
  const int tid = threadIdx.x;
  const int g = 4 * n <= NT ? 4 : 1;              // threads per logit (uniform)
  const int i = tid / g, part = tid % g;
  const int n4 = (n + 3) & ~3;                     // whole vectors of four entries
  const int per = ((n4 / 4 + g - 1) / g) * 4;      // entries per part, a multiple of 4
  const int j0 = part * per, j1 = min(j0 + per, n4);
  const uint32_t ki = i < n ? L.key[i] : 0xFFFFFFFFu;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int j = j0; j < j1; j += 4) {               // lanes of a quad read the same entries
    const uint4 k4 = *reinterpret_cast<const uint4*>(&L.key[j]);
    const double2 w01 = *reinterpret_cast<const double2*>(&L.w[j]);
    const double2 w23 = *reinterpret_cast<const double2*>(&L.w[j + 2]);
    s[0] += (k4.x >= ki && j < n) ? w01.x : 0.0;
    s[1] += (k4.y >= ki && j + 1 < n) ? w01.y : 0.0;
    s[2] += (k4.z >= ki && j + 2 < n) ? w23.x : 0.0;
    s[3] += (k4.w >= ki && j + 3 < n) ? w23.y : 0.0;
  }
  double t = (s[0] + s[1]) + (s[2] + s[3]);
  if (g == 4) {                                    // the quad's parts, in order
    const double t1 = __shfl_xor(t, 1), t2 = __shfl_xor(t, 2), t3 = __shfl_xor(t, 3);
    const int q = part;
    const double a0 = q == 0 ? t : q == 1 ? t1 : q == 2 ? t2 : t3;     // part 0
    const double a1 = q == 1 ? t : q == 0 ? t1 : q == 3 ? t2 : t3;     // part 1
    const double a2 = q == 2 ? t : q == 3 ? t1 : q == 0 ? t2 : t3;     // part 2
    const double a3 = q == 3 ? t : q == 2 ? t1 : q == 1 ? t2 : t3;     // part 3
    t = (a0 + a1) + (a2 + a3);
  }
  if (i < n && part == 0 && above + t >= target) atomicMax(&L.kcut, ki);
  __syncthreads();
  const uint32_t k = L.kcut ? L.kcut : (n > 0 ? L.kmin : 0u);
  __syncthreads();
  return k;
}

// ----------------------------------------------------- bf16 one pass ---
// A bf16 logit is one of at most 65536 values, so a histogram with a
// counter per distinct value holds a row exactly, and needs no reference
// value before the pass: one pass over the row fills it, and the row's
// largest value, the top-k cut, and the top-p cut with its kept mass (a
// value's mass is its count times its weight 2^(l c - Mref), in fp64) are
// read off descending scans of the counters. Each magnitude in
// [2^-16, 2^16) has a counter per sign, indexed by its bits (32 binades of
// 128 values); the word of a counter holds the count of the row's even
// positions in its low half and of the odd ones in its high half, so each
// logit adds a constant (a total that does not come to V shows a carry
// between the halves: the general search then runs). Magnitudes below
// 2^-16 ("tiny") share one count with the sums of their values, squares
// and cubes, which give their mass 2^-Mref sum e^x, x = l c ln 2,
// |x| < 2^-16 c ln 2, to O(x^4). -inf logits are counted apart (they weigh
// nothing). A row holding any other value outside the table (NaN, +inf,
// |l| >= 2^16), and a cut that falls among the tiny magnitudes, take the
// general search.

// Every 16-byte vector of a bf16 row once, raw: wave w of the workgroup
// streams chunks w, w + kWaves, ... with the next chunk's loads in flight
// while the current one is used (as in the row pass); pre() runs in every
// thread once the first loads are in flight; f(word, e) gets each
// 32-bit word (logits e and e + 1) once. Logits at or past V read as bf16
// -inf (0xFF80).
template <bool kVec, class P, class F>
__device__ __forceinline__ void for_each_word_bf16(const char* row, int n_chunk, int V, P pre, F f) {
  constexpr int kCE = Chunk<kBF16>::kElems;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int n_full = V / kCE;
  auto use = [&](ChunkRaw& r, int ch) {
#pragma unroll
    for (int j = 0; j < kLoadsPerLane; ++j) {
      const int64_t e = (int64_t)ch * kCE + (int64_t)(j * 64 + lane) * 8;
      f(r.v[j].x, e);
      f(r.v[j].y, e + 2);
      f(r.v[j].z, e + 4);
      f(r.v[j].w, e + 6);
    }
  };
  int ch = wave;
  const int ch_end = kVec ? n_full : 0;
  ChunkRaw ra, rb;
  const bool piped = ch < ch_end;
  if (piped) issue_chunk<kBF16>(row, (int64_t)ch * kCE, ra);
  pre();
  if (piped) {
    while (true) {
      int nx = ch + kWaves;
      bool more = nx < ch_end;
      issue_chunk<kBF16>(row, (int64_t)(more ? nx : ch) * kCE, rb);
      use(ra, ch);
      ch = nx;
      if (!more) break;
      nx = ch + kWaves;
      more = nx < ch_end;
      issue_chunk<kBF16>(row, (int64_t)(more ? nx : ch) * kCE, ra);
      use(rb, ch);
      ch = nx;
      if (!more) break;
    }
  }
  for (; ch < n_chunk; ch += kWaves) {
    ChunkRaw r;
    load_chunk_checked<kBF16, kVec>(row, (int64_t)ch * kCE, V, r);
    use(r, ch);
  }
}


// One lane's tallies of the logits outside the table.
struct HistRare {
  float s1, s2, s3;                                // sums of l, l^2, l^3 over tiny magnitudes
  unsigned n, ninf, kmax;                          // tiny count, -inf count, largest tiny order key
  bool big;                                        // NaN, +inf or |l| >= 2^16
  uint32_t undo_p, undo_n;                         // what they added to each sign's last word
  __device__ __forceinline__ void add(uint32_t h) {
    if ((h & 0x7FFFu) < kHMagLo) {
      const float v = __uint_as_float(h << 16);
      s1 += v;
      s2 += v * v;
      s3 += v * v * v;
      ++n;
      kmax = max(kmax, order_key(v));
    } else if (h == 0xFF80u) {
      ++ninf;
    } else {
      big = true;
    }
  }
};

// One pass over a bf16 row into the counters (zeroed, with the tallies and
// pick slots, while the first loads are in flight), then the lanes'
// tallies folded into L. Both logits of a 32-bit word are indexed at once
// in 16-bit lanes: magnitude - kHMagLo, wrapping below the table, clamped
// to the table's last position, so that a value outside the table (tiny,
// -inf, NaN, |l| >= 2^16) costs no extra instruction on the common path;
// one compare finds the words holding one, whose lanes take the rare path
// and later take their counts back out of the last words.
typedef unsigned short HU16x2 __attribute__((ext_vector_type(2)));
template <bool kVec>
__device__ __forceinline__ void hist_pass(const char* row, int n_chunk, int V, SelLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  HistRare t{0.f, 0.f, 0.f, 0u, 0u, 0u, false, 0u, 0u};
  auto zero = [&]() {
    uint4* z = reinterpret_cast<uint4*>(L.hcnt);
    for (int j = threadIdx.x; j < kHWords / 4; j += kThreads) z[j] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) {
      L.tiny_n = 0u;
      L.ninf_n = 0u;
      L.tiny_max = 0u;
      L.big = 0;
    }
    if (threadIdx.x < 64) L.tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
    __syncthreads();
  };
  char* const base = reinterpret_cast<char*>(L.hcnt);
  for_each_word_bf16<kVec>(row, n_chunk, V, zero, [&](uint32_t w, int64_t) {
    constexpr unsigned short lo = kHMagLo, top = kHBins - 1;
    const HU16x2 d = __builtin_bit_cast(HU16x2, w & 0x7FFF7FFFu) - HU16x2{lo, lo};
    const HU16x2 e = __builtin_elementwise_min(d, HU16x2{top, top});
    // byte offsets of the two words: 4 e, plus the negative table's 0x4000
    const uint32_t a = __builtin_bit_cast(uint32_t, HU16x2(e << (unsigned short)2)) | ((w >> 1) & 0x40004000u);
    atomicAdd(reinterpret_cast<uint32_t*>(base + (a & 0xFFFFu)), 1u);
    atomicAdd(reinterpret_cast<uint32_t*>(base + (a >> 16)), 0x10000u);
    if (__builtin_bit_cast(uint32_t, e) != __builtin_bit_cast(uint32_t, d)) {
      if (e.x != d.x) {
        if (w & 0x8000u) t.undo_n += 1u;
        else t.undo_p += 1u;
        t.add(w & 0xFFFFu);
      }
      if (e.y != d.y) {
        if (w & 0x80000000u) t.undo_n += 0x10000u;
        else t.undo_p += 0x10000u;
        t.add(w >> 16);
      }
    }
  });
  const float s1 = wave_sum_all(t.s1), s2 = wave_sum_all(t.s2), s3 = wave_sum_all(t.s3);
  if (lane == 0) {
    L.tiny_w[wave][0] = s1;
    L.tiny_w[wave][1] = s2;
    L.tiny_w[wave][2] = s3;
  }
  if (t.n) {
    atomicAdd(&L.tiny_n, t.n);
    atomicMax(&L.tiny_max, t.kmax);
  }
  if (t.ninf) atomicAdd(&L.ninf_n, t.ninf);
  if (t.big) L.big = 1;
  if (t.undo_p) atomicSub(&L.hcnt[kHOff + kHBins - 1], t.undo_p);
  if (t.undo_n) atomicSub(&L.hcnt[kHOff + kHNeg + kHBins - 1], t.undo_n);
  __syncthreads();
}

// Ordered positions, largest value first: [0, kHBins) the positive table
// from just below 2^16 down to 2^-16, kHBins the tiny magnitudes, then the
// negative table from -2^-16 down, and last (kHOrd - 1) -inf.
// The logit value of an ordered position (not the tiny one).
__device__ __forceinline__ float hist_value(int o) {
  if (o < kHBins) return __uint_as_float((kHMagLo + (uint32_t)(kHBins - 1 - o)) << 16);
  if (o < kHOrd - 1) return __uint_as_float((0x8000u | (kHMagLo + (uint32_t)(o - kHBins - 1))) << 16);
  return kNegInf;
}

// One thread's run of ordered positions: kHPerT table counters in order
// (a quarter of one binade, so consecutive values differ by the binade's
// spacing u and their weights by the factor 2^(-u c)), then for thread
// kThreads / 2 - 1 the tiny position and for the last thread the -inf one.
constexpr int kHPerT = 2 * kHBins / kThreads;
static_assert(kHPerT == 32 && kHBins % kHPerT == 0, "a run is a quarter binade");
static_assert(kThreads == 4 * 64 && kWaves == 4, "two waves per table");
static_assert(kHOff % 4 == 0 && kHNeg % 4 == 0 && kHWords % 4 == 0, "16-byte aligned runs");
struct HBlock {
  uint32_t n[kHPerT];                              // counts
  int o0;                                          // ordered position of n[0]
  float v0, u;                                     // value of n[0], spacing
  unsigned nx;                                     // count of the extra position (0: none)
  int ox;                                          // its ordered position
};

__device__ __forceinline__ void hist_block_load(const SelLds& L, unsigned n_tiny, unsigned n_ninf, HBlock& hb) {
  const int t = threadIdx.x;
  // waves 0 and 1 hold the positive table, 2 and 3 the negative one: a
  // uniform branch, so that the runs' words are picked by constant indices
  const bool pos = __builtin_amdgcn_readfirstlane(t >> 6) < kWaves / 2;
  const int rel = pos ? kHBins - kHPerT * (t + 1) : kHPerT * (t - kThreads / 2);   // magnitude - kHMagLo
  const uint4* q = reinterpret_cast<const uint4*>(L.hcnt + kHOff + rel + (pos ? 0 : kHNeg));
  uint32_t w[kHPerT];
#pragma unroll
  for (int k = 0; k < kHPerT / 4; ++k) {
    const uint4 x = q[k];
    w[4 * k] = x.x;
    w[4 * k + 1] = x.y;
    w[4 * k + 2] = x.z;
    w[4 * k + 3] = x.w;
  }
  if (pos) {                                       // positive values: descending bits
#pragma unroll
    for (int j = 0; j < kHPerT; ++j) hb.n[j] = (w[kHPerT - 1 - j] & 0xFFFFu) + (w[kHPerT - 1 - j] >> 16);
  } else {
#pragma unroll
    for (int j = 0; j < kHPerT; ++j) hb.n[j] = (w[j] & 0xFFFFu) + (w[j] >> 16);
  }
  const uint32_t mag0 = kHMagLo + (uint32_t)(pos ? rel + kHPerT - 1 : rel);
  hb.o0 = pos ? kHPerT * t : kHBins + 1 + kHPerT * (t - kThreads / 2);
  hb.v0 = __uint_as_float(((pos ? 0u : 0x8000u) | mag0) << 16);
  hb.u = __uint_as_float(((mag0 & 0x7F80u) - (7u << 7)) << 16);   // 2^(e - 7)
  hb.nx = t == kThreads / 2 - 1 ? n_tiny : (t == kThreads - 1 ? n_ninf : 0u);
  hb.ox = t == kThreads / 2 - 1 ? kHBins : kHOrd - 1;
}

// The thread holding ordered position o.
__device__ __forceinline__ int hist_owner(int o) {
  if (o < kHBins) return o / kHPerT;
  if (o == kHBins) return kThreads / 2 - 1;
  if (o == kHOrd - 1) return kThreads - 1;
  return kThreads / 2 + (o - kHBins - 1) / kHPerT;
}

// Every thread passes its candidate position (INT_MAX: none) and the
// running sum there; returns the smallest candidate over the workgroup (-1:
// none), and its sum in *at (from L.scan, where each candidate leaves its
// own). Each wave's smallest candidate, found on the DPP network, goes to
// picks[wave] with one store: LDS atomics from every lane to one word queue
// behind the counting of the CU's other workgroups (measured: 2 us).
__device__ __forceinline__ int hist_pick(SelLds& L, int* picks, int mine, double mine_at, double* at) {
  if (mine != INT_MAX) L.scan[threadIdx.x] = mine_at;
  int m = mine;
  m = min(m, dpp_i<kDppXor1>(m));
  m = min(m, dpp_i<kDppXor2>(m));
  m = min(m, dpp_i<kDppHalfMirror>(m));
  m = min(m, dpp_i<kDppMirror>(m));
  m = min(min(__builtin_amdgcn_readlane(m, 0), __builtin_amdgcn_readlane(m, 16)),
          min(__builtin_amdgcn_readlane(m, 32), __builtin_amdgcn_readlane(m, 48)));
  if ((threadIdx.x & 63) == 0) picks[threadIdx.x >> 6] = m;
  __syncthreads();
  int o = picks[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) o = min(o, picks[w]);
  if (o == INT_MAX) return -1;
  *at = L.scan[hist_owner(o)];
  return o;
}

// 2^(d - 1/32) for d in [-1/16, 0] or so (a weight relative to the middle
// of its level-0 bucket): e^x, x = (d + 1/32) ln 2, |x| <= 0.0217, by its
// Taylor series to x^7 (the remainder is below 2e-18 of the value).
__device__ __forceinline__ double exp2_small(double d) {
  const double x = (d + 0.03125) * 0.69314718055994530942;
  double e = 1.0 / 5040.0;
  e = fma(e, x, 1.0 / 720.0);
  e = fma(e, x, 1.0 / 120.0);
  e = fma(e, x, 1.0 / 24.0);
  e = fma(e, x, 1.0 / 6.0);
  e = fma(e, x, 0.5);
  e = fma(e, x, 1.0);
  return fma(e, x, 1.0);
}

// The weight of level-0 bucket k's middle, 2^(-k/16 - 1/32), by which the
// scan scales the bucket's exp2_small sum.
__device__ __forceinline__ double bucket_scale(int k) { return exp2(-0.0625 * (double)k - 0.03125); }

// The cut for one criterion among the logits with key >= kfloor: the
// largest logit value t whose upper set holds at least `want` logits
// (kMass false) or `want` of their mass (kMass true). Returns the key of t,
// or 0 to keep them all. Logits below kfloor count as -inf. Every thread of
// the src.kNT-thread workgroup calls.
// Level 0 is one pass of straight-line work per logit: its bucket k and one
// LDS atomic, the count, or the weight relative to the bucket's middle,
// 2^(D + k / 16 + 1/32) (a short series, no table), which the scan scales
// back (bucket_scale); the last bucket (D < -64, -inf) adds no mass. The bucket
// holding the cut is collected (key and fp64 weight) and cut exactly
// (rank_cut, or the sort for more than NT logits); with more than kSelCap
// logits in it, the next level refines it.
template <bool kMass, class Src, class LT>
__device__ __forceinline__ uint32_t select_cut(const Src& src, LT& L, double cd, float mref, double want,
                                               uint32_t kfloor) {
  constexpr int NT = Src::kNT, last = kSelBuckets0 - 1;
  const int tid = threadIdx.x;
  int64_t parent = 0;
  double above = 0.0, target = want;
  for (int level = 0;; ++level) {
    const int nb = level == 0 ? kSelBuckets0 : kSelBuckets;
    for (int i = tid; i < nb; i += NT) {
      if (!kMass || level > 0) L.cnt[i] = 0u;
      if (kMass) L.mass[i] = 0.0;
    }
    __syncthreads();
    if (level == 0) {                              // every logit lands in a bucket
      // the last one (D < -64, -inf, below kfloor) is not tallied: it
      // weighs nothing, and a count cut there keeps the whole row, as
      // does a target that no bucket's running count reaches; its atomics
      // would all hit one word (rows with many -inf logits)
      src.each([&](float l, int64_t) {
        const double D = order_key(l) >= kfloor ? (double)l * cd - (double)mref : -INFINITY;
        const int bk = sel_bucket(D, 0, 0);
        if (bk < last) {
          if (kMass) atomicAdd(&L.mass[bk], exp2_small(fma((double)bk, 0.0625, D)));
          else       atomicAdd(&L.cnt[bk], 1u);
        }
      });
    } else {                                       // only those of the parent bucket
      src.each([&](float l, int64_t) {
        const double D = order_key(l) >= kfloor ? (double)l * cd - (double)mref : -INFINITY;
        const int bk = sel_bucket(D, level, parent);
        if (bk >= 0) {
          atomicAdd(&L.cnt[bk], 1u);
          if (kMass) atomicAdd(&L.mass[bk], exp2_weight(D, L.tab));
        }
      });
    }
    __syncthreads();
    // a scan over the buckets, thread t taking buckets t per ... t per + per - 1
    const int per = nb >= NT ? nb / NT : 1;
    auto value = [&](int e) {
      if (!kMass) return (double)L.cnt[e];
      return level == 0 ? L.mass[e] * bucket_scale(e) : L.mass[e];
    };
    double loc = 0.0;
    for (int j = 0; j < per; ++j) {
      const int e = tid * per + j;
      if (e < nb) loc += value(e);
    }
    if (tid == 0) L.sel = INT_MAX;
    double excl, all;
    wg_scan<NT>(loc, L.wtot, &excl, &all);
    if (level == 0 && kMass) target = want * all;
    // the thread whose buckets hold the crossing leaves the sum before it
    double run = above + excl;
    for (int j = 0; j < per; ++j) {
      const int e = tid * per + j;
      if (e >= nb) break;
      const double v = value(e);
      if (run + v >= target) {
        atomicMin(&L.sel, e);
        L.scan[tid] = run;
        break;
      }
      run += v;
    }
    __syncthreads();
    const int sel = L.sel;
    if (sel == INT_MAX || (level == 0 && sel == last)) return 0u;   // keep all
    above = L.scan[sel / per];                     // the mass (or count) above bucket sel
    if (tid == 0) {
      L.n = 0;
      L.kcut = 0u;
      L.kmin = 0xFFFFFFFFu;
    }
    __syncthreads();
    // collect the bucket (its smallest key too)
    src.each([&](float l, int64_t) {
      const uint32_t k = order_key(l);
      const double D = k >= kfloor ? (double)l * cd - (double)mref : -INFINITY;
      if (sel_bucket(D, level, parent) != sel) return;
      atomicMin(&L.kmin, k);
      const int slot = atomicAdd(&L.n, 1);
      if (slot < kSelCap) {
        L.key[slot] = k;
        L.w[slot] = kMass ? exp2_weight(D, L.tab) : 1.0;
      }
    });
    __syncthreads();
    const int n = L.n;
    if (n <= NT) return rank_cut<NT>(L, n, above, target);
    if (n <= kSelCap) return scan_collected<NT>(L, n, above, target);
    if (level + 1 == kSelLevels) {
      // more than kSelCap logits within 2^-20 / 16 of one log2 weight: keep
      // that whole bucket (its smallest key)
      const uint32_t k = L.kmin;
      __syncthreads();
      return k;
    }
    parent = level == 0 ? sel : parent * kSelBuckets + sel;
    __syncthreads();
  }
}

constexpr int kRThreads = 1024;
constexpr int kRWaves = kRThreads / 64;
constexpr int kRCap = 32768;                       // logits: 128 KiB of LDS
constexpr int kRVecs = kRCap / 4 / kRThreads;      // 16-byte loads per thread
static_assert(kSelCap % kRThreads == 0 && kSelBuckets0 % kRThreads == 0, "whole shares per thread");

struct alignas(16) RSelLds {
  float4 row[kRCap / 4];
  union {                                          // the histogram, then the collected logits
    struct {
      unsigned cnt[kSelBuckets0];
      double mass[kSelBuckets0];
      double scan[kRThreads];                      // per thread: the sum before its pick
    };
    struct {
      uint32_t key[kSelCap];
      double w[kSelCap];
    };
  };
  double tab[64];                                  // 2^(j / 64)
  double wtot[kRWaves];
  float wsum[kRWaves];
  int n, sel;
  uint32_t kfloor, kcut, kmin;
};

// select_cut for a row held in LDS by a workgroup of kRThreads (one bucket
// of level 0 per thread), with the passes written out so that each is
// straight-line work per logit, without waits: the level-0 histogram (the
// bucket from the fp32 log2 weight, the weight relative to the bucket from
// the fp64 one); the scan, where the one thread whose range holds the
// crossing names the bucket; then the bucket's logits, which each thread
// marks in a bit mask, places by a scan of the counts, and writes out (key,
// fp64 weight) in a loop over its bits; and rank_cut. More than kSelCap
// logits in the bucket: select_cut, from the start.
template <bool kMass, int NT, int NV>
__device__ __forceinline__ uint32_t lds_select_cut(const LdsRow<NT, NV>& src, RSelLds& L, float c, double cd,
                                                   float mref, double want, uint32_t kfloor) {
  static_assert(NT == kSelBuckets0 && 4 * NV <= 32, "a bucket per thread; a bit per logit");
  constexpr int last = kSelBuckets0 - 1;
  const int tid = threadIdx.x;
  if (kMass) L.mass[tid] = 0.0;
  else       L.cnt[tid] = 0u;
  if (tid == 0) {
    L.sel = INT_MAX;
    L.kcut = 0u;
    L.kmin = 0xFFFFFFFFu;
  }
  __syncthreads();
  float4 q[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * NT + tid;
    q[j] = v < src.n_vec ? src.vec[v] : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
  }
  auto logit = [&](int i) {                        // static i: logit i of this thread
    const float4& v = q[i >> 2];
    return (i & 3) == 0 ? v.x : (i & 3) == 1 ? v.y : (i & 3) == 2 ? v.z : v.w;
  };
  // the bucket from the fp32 log2 weight (any monotone map will do, the
  // same in every pass; this one lies within 1e-4 of the fp64 one); the
  // weight from the fp64 one
  auto bucket = [&](float l) {
    const float t = -16.f * fmaf(l, c, -mref);
    const int bk = t < (float)last ? (t > 0.f ? (int)t : 0) : last;   // also -inf and NaN
    return order_key(l) >= kfloor ? bk : last;
  };
  // The last bucket (D < -64, -inf, below kfloor, and the slots past V) is
  // not tallied: it weighs nothing, and a count cut there keeps the whole
  // row, as does a target that no bucket's running count reaches. Its
  // atomics would all hit one word (a row of 1000 logits: 31,768 padding
  // slots, 51 us per call).
#pragma unroll
  for (int i = 0; i < 4 * NV; ++i) {
    const float l = logit(i);
    const int bk = bucket(l);
    if (bk < last) {
      if (kMass) {
        const double D = (double)l * cd - (double)mref;
        atomicAdd(&L.mass[bk], exp2_small(fma((double)bk, 0.0625, D)));
      } else {
        atomicAdd(&L.cnt[bk], 1u);
      }
    }
  }
  __syncthreads();
  const double v = kMass ? L.mass[tid] * bucket_scale(tid) : (double)L.cnt[tid];
  double excl, all;
  const double incl = wg_scan<NT>(v, L.wtot, &excl, &all);
  const double target = kMass ? want * all : want;
  if ((tid == 0 || excl < target) && target <= incl) {   // at most one thread
    L.sel = tid;
    L.scan[0] = excl;
  }
  __syncthreads();
  const int sel = L.sel;
  if (sel == INT_MAX || sel == last) return 0u;    // keep all
  const double above = L.scan[0];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 4 * NV; ++i) m |= (bucket(logit(i)) == sel ? 1u : 0u) << i;
  double ox, n_all;
  const int off = (int)(wg_scan<NT>((double)__builtin_popcount(m), L.wtot, &ox, &n_all) - __builtin_popcount(m));
  const int n = (int)n_all;
  if (n > kSelCap) return select_cut<kMass>(src, L, cd, mref, want, kfloor);
  const float* row = reinterpret_cast<const float*>(src.vec);
  uint32_t kmin = 0xFFFFFFFFu;
  for (int slot = off; m; ++slot) {
    const int i = __builtin_ctz(m);
    m &= m - 1u;
    const float l = row[(int64_t)((i >> 2) * NT + tid) * 4 + (i & 3)];
    const uint32_t k = order_key(l);
    const double D = k >= kfloor ? (double)l * cd - (double)mref : -INFINITY;
    L.key[slot] = k;
    L.w[slot] = kMass ? exp2_weight(D, L.tab) : 1.0;
    kmin = min(kmin, k);
  }
  if (kmin != 0xFFFFFFFFu) atomicMin(&L.kmin, kmin);
  __syncthreads();
  if (n <= NT) return rank_cut<NT>(L, n, above, target);
  return scan_collected<NT>(L, n, above, target);
}

template <bool kMass, class Src, class LT>
__device__ __forceinline__ uint32_t row_cut(const Src& src, LT& L, float, double cd, float mref, double want,
                                            uint32_t kfloor) {
  return select_cut<kMass>(src, L, cd, mref, want, kfloor);
}
template <bool kMass, int NT, int NV>
__device__ __forceinline__ uint32_t row_cut(const LdsRow<NT, NV>& src, RSelLds& L, float c, double cd, float mref,
                                            double want, uint32_t kfloor) {
  return lds_select_cut<kMass>(src, L, c, cd, mref, want, kfloor);
}

// The general search's cut of one row (top-k, then top-p, each by
// select_cut) and its kept mass: the fp32 sum of the kept weights
// 2^(l c - mref), without token xe (a one-hot draft's, as the row pass
// leaves it out; -1: none). L.tab must hold 2^(j / 64), j < 64.
template <class Src, class LT>
__device__ __forceinline__ void general_cut(const Src& src, int V, LT& L, float c, double cd, float mref, int tk,
                                            float tp, int xe, float* thr_out, float* s_out) {
  constexpr int NW = Src::kNT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t cut = 0u;
  if (tk > 0 && tk < V) cut = row_cut<false>(src, L, c, cd, mref, (double)tk, 0u);
  if (tp < 1.f) {                                  // NaN compares false: off
    const uint32_t cp = row_cut<true>(src, L, c, cd, mref, (double)tp, cut);
    if (cp) cut = cp;
  }
  const float thr = cut ? key_value(cut) : kNegInf;
  float sm = 0.f;
  src.each([&](float l, int64_t e) {
    sm += (l >= thr && e != xe) ? fast_exp2(fmaf(l, c, -mref)) : 0.f;
  });
  sm = wave_sum_all(sm);
  __syncthreads();                                 // earlier readers of L.wsum are done
  if (lane == 0) L.wsum[wave] = sm;
  __syncthreads();
  float v[NW];                                     // the wave sums, added pairwise
#pragma unroll
  for (int w = 0; w < NW; ++w) v[w] = L.wsum[w];
#pragma unroll
  for (int h = 1; h < NW; h <<= 1)
#pragma unroll
    for (int w = 0; w + h < NW; w += 2 * h) v[w] += v[w + h];
  *s_out = v[0];
  *thr_out = thr;
}

// fp32 rows, after the row pass: per row the cut (general_cut) and the kept
// mass, as a RowFilter for the filtered rule.
// Four workgroups per CU: the passes are latency-bound, and the occupancy
// this buys outweighs the few registers it spills.
template <int MODE, int DT, bool kVec>
__global__ __launch_bounds__(kThreads, 4) void sv_select_kernel(Args A) {
  __shared__ SelLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rowg = blockIdx.x;
  const int b = rowg / A.rows, r = rowg % A.rows;
  const Req rq = request(A, b);
  // Rows past a certain rejection are never drawn from (one-hot drafts,
  // top-k off): the kept mass of a top-p cut is at least top_p, so the
  // filtered p'(x) <= p(x) / top_p, and u * top_p >= p(x) (with a margin for
  // fp32 rounding) rejects position j whatever the cut; the rule stops at or
  // before it. p(x) is the unfiltered probability from the row pass; a
  // draft token outside [0, V) is always rejected. When the caller takes
  // only tokens (no p / q outputs) such a row needs no cut.
  bool past_reject = false;
  if constexpr (MODE == kOneHot) {
    if (r > 0 && r <= A.K) {
      __shared__ int s_skip;
      if (wave == 0) {
        const int tk0 = A.top_k ? A.top_k[b] : 0;
        const float tp0 = A.top_p ? A.top_p[b] : 1.f;
        const float tpe = (tp0 >= 1.f || tp0 != tp0) ? 1.f : tp0;   // filter off: p' = p
        const float T0 = A.temperature[b];
        const bool can = (tk0 <= 0 || tk0 >= A.V) && tpe > 0.f && T0 > 0.f && T0 < __builtin_inff();
        bool certain = false;
        if (can && lane < r) {
          const int j = lane;
          const int xj = A.tokens[(int64_t)b * A.K + j];
          if ((unsigned)xj >= (unsigned)A.V) {
            certain = true;
          } else {
            const int64_t rj = (int64_t)b * A.rows + j;
            float M = kNegInf, S = 0.f;
            for (int w = 0; w < A.wpr; ++w) {
              const float2 v = A.wpart[rj * A.wpr + w];
              ms_merge(M, S, v.x, v.y);
            }
            const float cj = kLog2e / T0, lx = A.gath[rj];
            const float Mx = fmaxf(M, lx * cj);
            const float Sx = (M == kNegInf) ? 0.f : S * fast_exp2(M - Mx);
            const float e = (Mx != kNegInf) ? fast_exp2(fmaf(lx, cj, -Mx)) : 0.f;
            const float St = Sx + e;
            const float pj = St > 0.f ? e / St : 0.f;
            const float u = A.unif[(int64_t)b * A.R + j].x;
            certain = u * tpe >= pj * 1.0001f + 1e-30f;
          }
        }
        const bool skip = __ballot(certain) != 0ull;
        if (lane == 0) s_skip = skip ? 1 : 0;
      }
      __syncthreads();
      past_reject = s_skip != 0;
      if (past_reject && !A.out_p && !A.out_q) return;
    }
  }
  const char* row = row_ptr(A, rq, r);
  const float T = A.temperature[b];
  // the row's largest scaled logit, from the row pass (which leaves a
  // one-hot draft token out of its sums)
  float m = kNegInf;
  for (int w = tid; w < A.wpr; w += kThreads) m = fmaxf(m, A.wpart[(int64_t)rowg * A.wpr + w].x);
  m = wave_max_all(m);
  if (lane == 0) L.wsum[wave] = m;
  if (tid < 64) L.tab[tid] = exp2((double)tid / 64.0);
  __syncthreads();
  float mref = fmaxf(fmaxf(L.wsum[0], L.wsum[1]), fmaxf(L.wsum[2], L.wsum[3]));
  const float c = kLog2e / T;
  int xe = -1;
  if (MODE == kOneHot && r < A.K) {
    xe = A.tokens[(int64_t)b * A.K + r];
    if ((unsigned)xe < (unsigned)A.V) mref = fmaxf(mref, A.gath[rowg] * c);
    else xe = -1;
  }
  if (!(T > 0.f && T < __builtin_inff()) || mref == kNegInf || mref != mref) {
    if (tid == 0) A.rf[rowg] = RowFilter{kNegInf, kNegInf, 0.f, 0.f};
    return;
  }
  const double cd = 1.4426950408889634 / (double)T;
  const int tk = A.top_k ? A.top_k[b] : 0;
  const float tp = A.top_p ? A.top_p[b] : 1.f;
  float thr, s;
  general_cut(StreamRow<DT, kVec>{row, A.n_chunk, A.V}, A.V, L, c, cd, mref, tk, tp, xe, &thr, &s);
  if (tid == 0) A.rf[rowg] = RowFilter{mref, thr, s, 0.f};
}

// fp32 rows of at most kRCap logits, one workgroup of kRThreads per row and
// no row pass before it: the workgroup copies its row to LDS (every load
// in flight at once; the copy and the sort's entries fill most of the CU's
// 160 KiB), and finds the row's largest value, its cuts and kept mass there
// (general_cut, each of its passes over LDS), as a RowFilter; also the
// row's draft-token logit and (row 0's workgroup) the request's uniforms,
// which the row pass draws on unfiltered calls.
template <int MODE, bool kVec>
__global__ __launch_bounds__(kRThreads) void sv_rselect_kernel(Args A) {
  __shared__ RSelLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rowg = blockIdx.x;
  const int b = rowg / A.rows, r = rowg % A.rows;
  const int V = A.V, n_vec = (V + 3) / 4;
  const Req rq = request(A, b);
  const char* row = row_ptr(A, rq, r);
  float4 x[kRVecs];
#pragma unroll
  for (int j = 0; j < kRVecs; ++j) {
    const int v = j * kRThreads + tid;
    const int64_t e0 = (int64_t)v * 4;
    if (kVec && e0 + 4 <= V) {
      x[j] = *reinterpret_cast<const float4*>(row + e0 * 4);
    } else {
      float q[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = e0 + k < V ? load_one<kF32>(row, e0 + k) : kNegInf;
      x[j] = make_float4(q[0], q[1], q[2], q[3]);
    }
  }
  auto draw_uniforms = [&]() {
    if (r == 0 && wave == 0 && lane < A.R) {
      const Philox4 rnd = philox4x64_10((uint64_t)lane, (uint64_t)b, A.offset, 0ull, A.seeds[b], 0ull);
      A.unif[(int64_t)b * A.R + lane] = make_float2(top24(rnd.w0), top24(rnd.w1));
    }
  };
  // this row's draft token (target rows 0..K-1, draft rows)
  const int i = r < A.R ? r : r - A.R;
  int xt = i < rq.k ? A.tokens[rq.x0 + i] : -1;
  if ((unsigned)xt >= (unsigned)V) xt = -1;
  const int xe = MODE == kOneHot ? xt : -1;        // left out of a one-hot row's sums
  const float T = A.temperature[b];
  float m = kNegInf;
#pragma unroll
  for (int j = 0; j < kRVecs; ++j) {
    if (j * kRThreads + tid < n_vec) L.row[j * kRThreads + tid] = x[j];
    m = fmaxf(m, fmaxf(fmaxf(x[j].x, x[j].y), fmaxf(x[j].z, x[j].w)));
  }
  m = wave_max_all(m);
  if (lane == 0) L.wsum[wave] = m;
  if (tid < 64) L.tab[tid] = exp2((double)tid / 64.0);
  __syncthreads();
  float lmax = kNegInf;
#pragma unroll
  for (int w = 0; w < kRWaves; ++w) lmax = fmaxf(lmax, L.wsum[w]);
  const float c = kLog2e / T;
  const float mref = lmax * c;
  float thr = kNegInf, s = 0.f, mr = kNegInf;
  if (T > 0.f && T < __builtin_inff() && mref != kNegInf && mref == mref) {
    const double cd = 1.4426950408889634 / (double)T;
    const int tk = A.top_k ? A.top_k[b] : 0;
    const float tp = A.top_p ? A.top_p[b] : 1.f;
    general_cut(LdsRow<kRThreads, kRVecs>{L.row, n_vec}, V, L, c, cd, mref, tk, tp, xe, &thr, &s);
    mr = mref;
  }
  if (tid == 0) {
    A.rf[rowg] = RowFilter{mr, thr, s, 0.f};
    if (xt >= 0) A.gath[rowg] = reinterpret_cast<const float*>(L.row)[xt];
  }
  draw_uniforms();
}

// bf16 rows, one workgroup per row and no row pass before it: the one-pass
// histogram, then the row's largest value, its cuts and kept mass, as a
// RowFilter; also the row's draft-token logit, and (row 0's workgroup) the
// request's uniforms, which the row pass draws on unfiltered calls.
template <int MODE, bool kVec>
__global__ __launch_bounds__(kThreads, 4) void sv_hselect_kernel(Args A) {
  constexpr int kCE = Chunk<kBF16>::kElems;
  __shared__ SelLds L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rowg = blockIdx.x;
  const int b = rowg / A.rows, r = rowg % A.rows;
  const Req rq = request(A, b);
  const char* row = row_ptr(A, rq, r);
  // row 0's workgroup: the request's uniforms, by wave 0 once the others
  // are done (nothing here waits for them)
  auto draw_uniforms = [&]() {
    if (r == 0 && wave == 0 && lane < A.R) {
      const Philox4 rnd = philox4x64_10((uint64_t)lane, (uint64_t)b, A.offset, 0ull, A.seeds[b], 0ull);
      A.unif[(int64_t)b * A.R + lane] = make_float2(top24(rnd.w0), top24(rnd.w1));
    }
  };
  // this row's draft token (target rows 0..K-1, draft rows); its logit's
  // load stays in flight during the pass
  const int i = r < A.R ? r : r - A.R;
  int xt = i < rq.k ? A.tokens[rq.x0 + i] : -1;
  if ((unsigned)xt >= (unsigned)A.V) xt = -1;
  float lx = kNegInf;
  if (tid == 0 && xt >= 0) lx = load_one<kBF16>(row, xt);
  const int xe = MODE == kOneHot ? xt : -1;        // left out of a one-hot row's sums
  const float T = A.temperature[b];
  if (!(T > 0.f && T < __builtin_inff())) {
    if (tid == 0) {
      A.rf[rowg] = RowFilter{kNegInf, kNegInf, 0.f, 0.f};
      if (xt >= 0) A.gath[rowg] = lx;
    }
    draw_uniforms();
    return;
  }
  const float c = kLog2e / T;
  const double cd = 1.4426950408889634 / (double)T;
  const int tk = A.top_k ? A.top_k[b] : 0;
  const float tp = A.top_p ? A.top_p[b] : 1.f;

  hist_pass<kVec>(row, A.n_chunk, A.V, L);
  if (tid == 0 && xt >= 0) A.gath[rowg] = lx;

  const unsigned n_tiny = L.tiny_n;
  const unsigned n_ninf = L.ninf_n - (unsigned)((int64_t)A.n_chunk * kCE - A.V);   // less the padding
  bool general = L.big != 0;
  if (!general) {
    HBlock hb;
    hist_block_load(L, n_tiny, n_ninf, hb);
    uint32_t cl = hb.nx;                           // this run's count
#pragma unroll
    for (int j = 0; j < kHPerT; ++j) cl += hb.n[j];
    int j1 = kHPerT;                               // its first counted table position
#pragma unroll
    for (int j = kHPerT - 1; j >= 0; --j) j1 = hb.n[j] ? j : j1;
    int o_max, o_k = -1;
    double at;
    // the largest value: the first counted position
    o_max = hist_pick(L, L.sel_max, j1 < kHPerT ? hb.o0 + j1 : (hb.nx ? hb.ox : INT_MAX), 0.0, &at);
    // counts: the top-k cut, and the total (a carry between the halves of a
    // word, possible only when V / 2 > 65535, shows as a total other than V)
    const bool k_on = tk > 0 && tk < A.V;
    if (k_on || A.V > 2 * 65535) {
      double ce, ct;
      const double ci = wg_scan<kThreads, true>((double)cl, L.wtot, &ce, &ct);
      general = ct != (double)A.V;
      if (k_on && !general) {
        const double target = (double)tk;
        int mine = INT_MAX;
        if (ce < target && ci >= target) {         // exact: integer sums
          double run = ce;
#pragma unroll
          for (int j = 0; j < kHPerT; ++j) {
            run += (double)hb.n[j];
            if (mine == INT_MAX && hb.n[j] && run >= target) mine = hb.o0 + j;
          }
          if (mine == INT_MAX) mine = hb.ox;       // the extra position completes it
        }
        o_k = hist_pick(L, L.sel_k, mine, 0.0, &at);
      }
    }
    if (!general && (o_max < 0 || o_max == kHOrd - 1)) {   // nothing but -inf: no mass
      if (tid == 0) A.rf[rowg] = RowFilter{kNegInf, kNegInf, 0.f, 0.f};
      draw_uniforms();
      return;
    }
    if (o_k == kHOrd - 1) o_k = -1;                // the k-th largest is -inf: keep all
    if (!general && o_k != kHBins) {
      const float lmax = o_max == kHBins ? key_value(L.tiny_max) : hist_value(o_max);
      const float mref = lmax * c;
      const int o_lim = o_k >= 0 ? o_k : kHOrd - 1;   // positions past it weigh nothing
      // tiny magnitudes: 2^-mref sum (1 + x + x^2/2 + x^3/6), x = l cd ln 2
      double s1 = 0.0, s2 = 0.0, s3 = 0.0;
      for (int w = 0; w < kWaves; ++w) {
        s1 += (double)L.tiny_w[w][0];
        s2 += (double)L.tiny_w[w][1];
        s3 += (double)L.tiny_w[w][2];
      }
      const double a = cd * 0.69314718055994530942;
      const double m_tiny = exp2_weight(-(double)mref, L.tab) *
                            ((double)n_tiny + a * s1 + a * a * s2 * 0.5 + a * a * a * s3 * (1.0 / 6.0));
      const double mx = (hb.nx && hb.ox == kHBins && hb.ox <= o_lim) ? m_tiny : 0.0;
      // The run's mass. Its weights fall by the factor 2^(-u c) per
      // position: with the whole run below the cut limit and its weights
      // spanning at most 2^960, Horner's rule from the largest value down,
      // scaled by the smallest value's weight (at most the largest's, about
      // 1 or less); otherwise, per position from the first counted one.
      const double ucd = (double)hb.u * cd;
      const int lim = o_lim - hb.o0;               // positions j <= lim count
      double ml = 0.0;
      if (j1 < kHPerT && lim >= kHPerT - 1 && ucd * (kHPerT - 1) <= 960.0) {
        const double g = exp2_weight(ucd, L.tab);
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < kHPerT; ++j) acc = fma(acc, g, (double)hb.n[j]);
        ml = acc * exp2_weight((double)(hb.v0 - (float)(kHPerT - 1) * hb.u) * cd - (double)mref, L.tab);
      } else if (j1 < kHPerT && lim >= j1) {
        const double rr = exp2_weight(-ucd, L.tab);
        double w = exp2_weight((double)(hb.v0 - (float)j1 * hb.u) * cd - (double)mref, L.tab);
#pragma unroll
        for (int j = 0; j < kHPerT; ++j) {
          if (j >= j1) {
            ml += j <= lim ? (double)hb.n[j] * w : 0.0;
            w *= rr;
          }
        }
      }
      ml += mx;
      double me, zk;
      const double mi = wg_scan<kThreads, true>(ml, L.wtot2, &me, &zk);
      const bool p_on = tp < 1.f;                  // NaN compares false: off
      int o_p = -1;
      double at_p = 0.0;
      if (p_on) {
        const double target = fmax((double)tp * zk, __DBL_MIN__);
        int mine = INT_MAX;
        double mine_at = 0.0;
        // The run holding the crossing is walked by its thread's whole
        // wave, lane j at the run's position j: its count from the table,
        // its weight by its own exp2 (one thread walking 32 positions in a
        // dependent chain took 2.4 us on a CU busy with other rows). The
        // first position whose running mass reaches the target is the
        // cut; a sum that rounds short of the scan's takes the run's last
        // position of positive mass, then the tiny ones, as the sequential
        // walk did.
        const uint64_t cross = __ballot(me < target && mi >= target);
        if (cross) {                               // uniform within the wave
          const int c = __builtin_ctzll(cross);
          const int o0 = __builtin_amdgcn_readlane(hb.o0, c), j1c = __builtin_amdgcn_readlane(j1, c);
          const int limc = __builtin_amdgcn_readlane(lim, c), oxc = __builtin_amdgcn_readlane(hb.ox, c);
          const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hb.v0), c));
          const float uu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hb.u), c));
          const double mec = readlane_d(me, c), mic = readlane_d(mi, c), mxc = readlane_d(mx, c);
          const int j = lane;
          double x = 0.0;
          if (j < kHPerT && j >= j1c && j <= limc) {
            const int o = o0 + j;
            const uint32_t wd = L.hcnt[o < kHBins ? kHOff + (kHBins - 1 - o) : kHOff + kHNeg + (o - kHBins - 1)];
            const uint32_t n = (wd & 0xFFFFu) + (wd >> 16);
            if (n) x = (double)n * exp2_weight((double)(v0 - (float)j * uu) * cd - (double)mref, L.tab);
          }
          const double pre = wave_scan_incl_d(x);
          const uint64_t hit = __ballot(x > 0.0 && mec + pre >= target);
          int last = -1;
          double at = 0.0;
          if (hit) {
            const int h = __builtin_ctzll(hit);
            last = o0 + h;
            at = mec + readlane_d(pre, h);
          } else {
            const uint64_t any = __ballot(x > 0.0);
            double run = mec + readlane_d(pre, 63);
            if (any) last = o0 + 63 - __builtin_clzll(any);
            if (run < target && mxc > 0.0) {
              run += mxc;
              last = oxc;
            }
            at = run >= target ? run : mic;
          }
          if (lane == c && last >= 0) {
            mine = last;
            mine_at = at;
          }
        }
        o_p = hist_pick(L, L.sel_p, mine, mine_at, &at_p);
      }
      if (!(p_on && o_p == kHBins)) {              // a cut among the tiny magnitudes: general search
        int o_c = o_k;
        double kept = zk;
        if (p_on && o_p >= 0) {
          o_c = o_p;
          kept = at_p;
        }
        if (tid == 0) {
          const float thr = o_c >= 0 ? hist_value(o_c) : kNegInf;
          double sk = kept;
          if (xe >= 0 && lx >= thr) sk -= exp2_weight((double)lx * cd - (double)mref, L.tab);
          A.rf[rowg] = RowFilter{mref, thr, (float)fmax(sk, 0.0), 0.f};
        }
        draw_uniforms();
        return;
      }
    }
  }
  // the general search, with the row's largest logit from one more pass
  float m = kNegInf;
  for_each_logit<kBF16, kVec>(row, A.n_chunk, A.V, [&](float l, int64_t) { m = fmaxf(m, l); });
  m = wave_max_all(m);
  __syncthreads();
  if (lane == 0) L.wsum[wave] = m;
  __syncthreads();
  const float mref = fmaxf(fmaxf(L.wsum[0], L.wsum[1]), fmaxf(L.wsum[2], L.wsum[3])) * c;
  if (mref == kNegInf || mref != mref) {
    if (tid == 0) A.rf[rowg] = RowFilter{kNegInf, kNegInf, 0.f, 0.f};
    draw_uniforms();
    return;
  }
  float thr, s;
  general_cut(StreamRow<kBF16, kVec>{row, A.n_chunk, A.V}, A.V, L, c, cd, mref, tk, tp, xe, &thr, &s);
  if (tid == 0) A.rf[rowg] = RowFilter{mref, thr, s, 0.f};
  draw_uniforms();
}

// The rule on filtered rows, one wave per request: p_i(x_i) = w(x_i) / S'_i
// with the kept weights and sums of the select pass. A token still to be
// drawn from a filtered target row (a one-hot residual, the bonus token)
// is left to the caller: rc.draw = 1, with its position, uniform, the row's
// reference and cut, and the token to leave out.
// write_out: as for sample_tail (false: only return the decision, for the
// residual pass's other workgroups).
template <int DT, bool kVec, int MODE>
__device__ __forceinline__ Record filtered_tail(const Args& A, int b, bool write_out = true) {
  Record rc;
  rc.pending = 0;
  rc.draw = 0;
  const int lane = threadIdx.x & 63;
  const Req rq = request(A, b);
  const int K = A.K, V = A.V, R = A.R;
  const int64_t rowg0 = (int64_t)b * A.rows;
  int x = -1;
  float lx = kNegInf, ld = kNegInf;
  if (lane < K) {
    x = A.tokens[(int64_t)b * K + lane];
    lx = A.gath[rowg0 + lane];
    if (MODE == kExplicit) ld = A.gath[rowg0 + R + lane];
  }
  RowFilter fpr = RowFilter{kNegInf, kNegInf, 0.f, 0.f}, fqr = fpr;
  if (lane <= K) fpr = A.rf[rowg0 + lane];
  if (MODE == kExplicit && lane < K) fqr = A.rf[rowg0 + R + lane];
  const float T = A.temperature[b];
  float2 un = make_float2(0.f, 0.f);
  if (lane <= K) un = A.unif[(int64_t)b * R + lane];
  int32_t* otok = A.out_tokens + (int64_t)b * A.out_cols;
  if (!(T > 0.f && T < __builtin_inff())) {        // refused request
    if (!write_out) return rc;
    if (lane <= K) otok[lane] = -1;
    if (lane < K && A.out_p) A.out_p[(int64_t)b * K + lane] = 0.f;
    if (lane < K && A.out_q) A.out_q[(int64_t)b * K + lane] = 0.f;
    if (lane == 0) {
      A.out_len[b] = 0;
      if (MODE == kExplicit) A.rec[b].pending = 0;
    }
    return rc;
  }
  const float c = kLog2e / T;
  float p = 0.f, q = 0.f, lp = kNegInf, lq = kNegInf;
  if (lane < K) {
    const bool valid = (unsigned)x < (unsigned)V;
    const bool kept = valid && lx >= fpr.thr && fpr.mref != kNegInf;
    if (MODE == kOneHot) {
      const float e = kept ? fast_exp2(fmaf(lx, c, -fpr.mref)) : 0.f;
      const float St = fpr.s + e;                 // the sums leave x out
      p = St > 0.f ? e / St : 0.f;
      q = valid ? 1.f : 0.f;
    } else {
      const bool keptq = valid && ld >= fqr.thr && fqr.mref != kNegInf;
      const float dp = fmaf(lx, c, -fpr.mref), dq = fmaf(ld, c, -fqr.mref);
      const bool okp = kept && fpr.s > 0.f, okq = keptq && fqr.s > 0.f;
      p = okp ? fast_exp2(dp) / fpr.s : 0.f;
      q = okq ? fast_exp2(dq) / fqr.s : 0.f;
      lp = okp ? dp - __log2f(fpr.s) : kNegInf;
      lq = okq ? dq - __log2f(fqr.s) : kNegInf;
    }
    if (write_out && A.out_p) A.out_p[(int64_t)b * K + lane] = p;
    if (write_out && A.out_q) A.out_q[(int64_t)b * K + lane] = q;
  }
  const bool accept = MODE == kOneHot ? (un.x * q < p) : (__log2f(un.x) + lq < lp);
  const int rej = first_lane(lane < K && !accept);
  const int a = rej < 0 ? K : rej;
  if (write_out) {
    if (lane <= K && lane != a) otok[lane] = lane < a ? x : -1;
    if (lane == 0) A.out_len[b] = a + 1;
  }
  const float ua = lane_f(un.y, a);
  const float Ma = lane_f(fpr.mref, a), ta = lane_f(fpr.thr, a);
  if (MODE == kExplicit) {
    if (a < K) {
      rc.a = a; rc.pending = 1; rc.c = c; rc.u = ua;
      rc.Mp = Ma; rc.Sp = lane_f(fpr.s, a); rc.Mq = lane_f(fqr.mref, a); rc.Sq = lane_f(fqr.s, a);
      rc.tp = ta; rc.tq = lane_f(fqr.thr, a);
      if (write_out && lane == 0) A.rec[b] = rc;
      return rc;
    }
    if (write_out && lane == 0) A.rec[b].pending = 0;
    if (!write_out) return rc;                     // the bonus draw is the writer's
  }
  // the token at a is drawn from the filtered target row a (one-hot: without
  // x_a), by the caller's workgroup (filtered_draw)
  rc.draw = 1;
  rc.a = a;
  rc.c = c;
  rc.u = ua;
  rc.Mp = Ma;
  rc.tp = ta;
  rc.xe = (MODE == kOneHot && a < K) ? lane_i(x, a) : -1;
  return rc;
}

// Lane l's 64-byte run of logits c0 + l * E ... (E = 32 bf16 or 16 fp32) of
// a chunk wholly inside the row, as raw words of four 16-byte loads;
// raw_logit reads logit k of it.
template <int DT>
__device__ __forceinline__ void lane_run_raw(const char* row, int64_t c0, uint32_t (&wd)[16]) {
  constexpr int E = Chunk<DT>::kElems / 64;
  static_assert(E * Elem<DT>::kBytes == 64, "a lane's run is 64 bytes");
  const int64_t e0 = c0 + (int64_t)(threadIdx.x & 63) * E;
  const uint4* p = reinterpret_cast<const uint4*>(row + e0 * Elem<DT>::kBytes);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = p[q];
    wd[4 * q] = v.x;
    wd[4 * q + 1] = v.y;
    wd[4 * q + 2] = v.z;
    wd[4 * q + 3] = v.w;
  }
}

template <int DT>
__device__ __forceinline__ float raw_logit(const uint32_t (&wd)[16], int k) {
  if (DT == kBF16) return __uint_as_float((k & 1) ? (wd[k >> 1] & 0xFFFF0000u) : (wd[k >> 1] << 16));
  return __uint_as_float(wd[k]);
}

// Sums of the kept weights 2^(l c - M) (l >= thr, token xe left out) of
// chunks w, w + nw, ... of one row, published to out[chunk]; lane l sums
// the E consecutive logits of the chunk that the draw gives it. Each wave
// has the loads of G chunks in flight at once. One chunk at a time: with
// every request reading its row at once (B = 256, bf16 rows of 128256
// logits, 16 waves per request) the call took 99.5 us against 101.5 with
// one chunk in flight while another is summed and 102.2 with four in
// flight; the waves whose loads came back last then still had all their
// exponentials to do.
template <int DT, bool kVec, int G = 1>
__device__ __forceinline__ void kept_chunk_sums(const char* row, int n_chunk, int V, float c, float M, float thr, int xe,
                                                float* out, int w, int nw, bool to_lds = false) {
  constexpr int kCE = Chunk<DT>::kElems, E = kCE / 64;
  const int lane = threadIdx.x & 63;
  auto put = [&](int ch, float sm) {
    sm = wave_sum_all(sm);
    if (lane == 0) {
      if (to_lds) out[ch] = sm;
      else publish(out + ch, sm);
    }
  };
  // chunks wholly inside an aligned row: G at a time, raw 16-byte loads
  const int n_full = kVec ? V / kCE : 0;
  for (int ch0 = w; ch0 < n_full; ch0 += G * nw) {
    uint32_t wd[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int ch = ch0 + g * nw;
      if (ch < n_full) lane_run_raw<DT>(row, (int64_t)ch * kCE, wd[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int ch = ch0 + g * nw;
      if (ch >= n_full) break;
      const int64_t e0 = (int64_t)ch * kCE + (int64_t)lane * E;
      float sm = 0.f;
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const float x = raw_logit<DT>(wd[g], k);
        sm += (x >= thr && e0 + k != xe) ? fast_exp2(fmaf(x, c, -M)) : 0.f;
      }
      put(ch, sm);
    }
  }
  // the rest (the row's partial last chunk; every chunk of an unaligned
  // row), one at a time; chunk ch stays with wave ch mod nw
  for (int ch = n_full + (((w - n_full) % nw) + nw) % nw; ch < n_chunk; ch += nw) {
    const int64_t c0 = (int64_t)ch * kCE;
    float x[E];
    load_lane_run_all<DT, kVec, E>(row, c0, V, x);
    const int64_t e0 = c0 + (int64_t)lane * E;
    float sm = 0.f;
#pragma unroll
    for (int k = 0; k < E; ++k) sm += (x[k] >= thr && e0 + k != xe) ? fast_exp2(fmaf(x[k], c, -M)) : 0.f;
    put(ch, sm);
  }
}

// The token at rc.a of request b, drawn from its filtered target row (the
// kept weights; one-hot: without rc.xe) by nw waves of the calling
// workgroup, all of whose threads call when nw > 1: the chunk sums go to
// the row's workspace slice, then wave 0 finds the chunk and the token.
// Only the one row a request draws from is read. lds (nw > 1): room for
// kDrawLdsChunks sums in the workgroup's LDS, used when the row's chunks
// fit; wave 0 then reads them there rather than back from memory (C3 with
// top_p 0.95: about 1 us per call).
constexpr int kDrawLdsChunks = 2048;

template <int DT, bool kVec>
__device__ __forceinline__ void filtered_draw(const Args& A, int b, const Record& rc, int nw, float* lds = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const Req rq = request(A, b);
  const char* row = row_ptr(A, rq, rc.a);
  const bool in_lds = lds != nullptr && nw > 1 && A.n_chunk <= kDrawLdsChunks;
  float* fp = in_lds ? lds : A.fpart + ((int64_t)b * A.rows + rc.a) * A.n_chunk;
  kept_chunk_sums<DT, kVec>(row, A.n_chunk, A.V, rc.c, rc.Mp, rc.tp, rc.xe, fp, wave, nw, in_lds);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);                   // this wave's sums are in memory
  if (nw > 1) __syncthreads();
  if (wave != 0) return;
  int y = draw_from_partials<DT, kVec, false, true>(A, b, rq, rc.a, rc.c, rc.Mp, rc.xe, rc.u, rc.tp,
                                                    [&](int s) { return make_float2(rc.Mp, in_lds ? fp[s] : fetch(fp + s)); });
  if (y < 0) y = ((unsigned)rc.xe < (unsigned)A.V) ? rc.xe : 0;   // no kept mass: p_a's mode
  if (lane == 0) A.out_tokens[(int64_t)b * A.out_cols + rc.a] = y;
}

// One workgroup per request (one-hot drafts): wave 0 runs the filtered
// rule, then every wave sums the kept weights of the row the token is
// drawn from, per chunk, and wave 0 draws it (filtered_draw).
constexpr int kDrawThreads = 1024;
constexpr int kDrawWaves = kDrawThreads / 64;

template <int MODE, int DT, bool kVec>
__global__ __launch_bounds__(kDrawThreads) void sv_ftail_kernel(Args A) {
  __shared__ Record s_rc;
  __shared__ float s_sums[kDrawLdsChunks];
  const int b = blockIdx.x;
  if (threadIdx.x < 64) {
    const Record rc = filtered_tail<DT, kVec, MODE>(A, b);
    if (threadIdx.x == 0) s_rc = rc;
  }
  __syncthreads();
  const Record rc = s_rc;
  if (rc.draw) filtered_draw<DT, kVec>(A, b, rc, kDrawWaves, s_sums);
}

// ------------------------------------------------------ residual pass ---
// Explicit draft logits: for requests that stopped at a < K, chunk sums of
// max(0, p_a - q_a); the last workgroup of the request draws the token.
// kFilt: p_a and q_a are the top-k / top-p filtered rows (weights below a
// row's cut count as zero).
// kDecide: no tail launch came before; every workgroup of a request runs
// the rule itself (one wave, sample_tail on the row pass's results: the
// same decision in each), workgroup 0 writes the outputs or draws the bonus
// token, and the pass goes on for requests that rejected.
template <int DT, bool kVec, bool kMask, bool kFilt, bool kDecide>
__global__ __launch_bounds__(kThreads) void sv_residual_kernel(Args A) {
  constexpr int kCE = Chunk<DT>::kElems;
  __shared__ TailLds S;
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  const int wi = (int)(blockIdx.x % (unsigned)A.wpr);
  const int b = (int)(blockIdx.x / (unsigned)A.wpr);
  Record rc;
  if constexpr (kDecide) {
    __shared__ Record s_rc;
    if (wave == 0) {
      Record r0;
      if constexpr (kFilt) r0 = filtered_tail<DT, kVec, kExplicit>(A, b, wi == 0);
      else r0 = sample_tail<DT, kVec, kExplicit, kMask>(A, b, S, wi == 0);
      if (lane == 0) s_rc = r0;
    }
    __syncthreads();
    rc = s_rc;
    if constexpr (kFilt) {
      if (rc.draw) {                               // all accepted: the bonus token, by this workgroup
        filtered_draw<DT, kVec>(A, b, rc, kWaves);
        return;
      }
    }
  } else {
    rc = A.rec[b];
  }
  if (!rc.pending) return;
  const int a = rc.a;
  const float c = rc.c;
  const float ip = 1.f / rc.Sp, iq = 1.f / rc.Sq;
  const Req req = request(A, b);
  const char* rowp = row_ptr(A, req, a);
  const char* rowq = row_ptr(A, req, A.R + a);
  const uint32_t* mrow = kMask ? mask_row(A, b, a) : nullptr;
  const int c_lo = wi * A.cpw;
  const int c_hi = min(c_lo + A.cpw, A.n_chunk);

  constexpr int kPer = Elem<DT>::kPerVec;
  for (int ch = c_lo + wave; ch < c_hi; ch += kWaves) {
    const int64_t c0 = (int64_t)ch * kCE;
    ChunkRaw rp, rq;
    if (kVec && ch < A.n_full) {
      issue_chunk<DT>(rowp, c0, rp);
      issue_chunk<DT>(rowq, c0, rq);
    } else {
      load_chunk_checked<DT, kVec>(rowp, c0, A.V, rp);
      load_chunk_checked<DT, kVec>(rowq, c0, A.V, rq);
    }
    if constexpr (kMask) {                         // disallowed: p = q = 0, no residual
      MaskRaw mr;
      issue_mask<DT>(mrow, c0, A.mask_words, mr);
      apply_mask<DT>(rp, mr);
      apply_mask<DT>(rq, mr);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kLoadsPerLane; ++j)
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const float yp = raw_elem<DT>(rp, j, k), yq = raw_elem<DT>(rq, j, k);
        float wp = fast_exp2(fmaf(yp, c, -rc.Mp)) * ip, wq = fast_exp2(fmaf(yq, c, -rc.Mq)) * iq;
        if constexpr (kFilt) {
          wp = yp >= rc.tp ? wp : 0.f;
          wq = yq >= rc.tq ? wq : 0.f;
        }
        s += fmaxf(wp - wq, 0.f);
      }
    s = wave_sum_all(s);
    if (lane == 0) publish(A.res_part + (int64_t)b * A.n_chunk + ch, s);
  }
  if (!last_of_request(A.counters + b, (unsigned)A.wpr, &s_last)) return;
  if (wave != 0) return;                          // the draw is one wave's work

  constexpr int E = kCE / 64;
  const float* rpart = A.res_part + (int64_t)b * A.n_chunk;
  auto W = [&](int sg) { return fetch(rpart + sg); };
  int found;
  float t_in;
  const float Z = wave_locate(A.n_chunk, rc.u, W, &found, &t_in);
  int y = -1;
  if (Z > 0.f && found >= 0) {
    const int64_t c0 = (int64_t)found * kCE;
    float xp[E], xq[E], w[E];
    load_lane_run<DT, kVec, E>(rowp, c0, A.V, xp);
    load_lane_run<DT, kVec, E>(rowq, c0, A.V, xq);
    const uint32_t allow = kMask ? lane_mask_bits<E>(mrow, c0, A.mask_words) : ~0u;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      float wp = fast_exp2(fmaf(xp[k], c, -rc.Mp)) * ip, wq = fast_exp2(fmaf(xq[k], c, -rc.Mq)) * iq;
      if constexpr (kFilt) {
        wp = xp[k] >= rc.tp ? wp : 0.f;
        wq = xq[k] >= rc.tq ? wq : 0.f;
      }
      w[k] = ((allow >> k) & 1u) ? fmaxf(wp - wq, 0.f) : 0.f;
    }
    y = wave_pick<E>(w, c0, t_in);
  }
  if (y < 0) {
    // p_a and q_a agree everywhere: draw from p_a
    if constexpr (kFilt) {
      Record d = rc;
      d.xe = -1;
      filtered_draw<DT, kVec>(A, b, d, 1);         // this wave alone
      return;
    } else {
      y = draw_softmax_row<DT, kVec, kMask>(A, b, req, a, c, rc.Mp, -1, rc.u, S, false);
    }
    if (y < 0) y = 0;
  }
  if (lane == 0) A.out_tokens[(int64_t)b * A.out_cols + a] = y;
}

// Filtered verification with draft logits on fp32 rows of at most
// kRes1Chunks chunks: one workgroup of kDrawThreads per request. Wave 0 runs the
// filtered rule and writes the outputs; the bonus token is drawn by all 16
// waves (filtered_draw). For a request that stopped at a < K every wave sums
// max(0, p'_a - q'_a) over its chunks of the stop row pair into LDS (two
// chunks' loads of both rows in flight), and wave 0 finds the chunk and the
// token: the chunk sums never leave the workgroup (no publish, no ticket).
// Unfiltered calls keep the residual pass of several workgroups per request,
// whose bonus draw reuses the row pass's chunk sums.
constexpr int kRes1Chunks = 4 * kDrawWaves;

template <int DT, bool kVec>
__global__ __launch_bounds__(kDrawThreads) void sv_fresidual_kernel(Args A) {
  constexpr int kCE = Chunk<DT>::kElems, kPer = Elem<DT>::kPerVec, E = kCE / 64;
  __shared__ Record s_rc;
  __shared__ float s_part[kRes1Chunks];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int b = blockIdx.x;
  if (wave == 0) {
    const Record r0 = filtered_tail<DT, kVec, kExplicit>(A, b, true);
    if (lane == 0) s_rc = r0;
  }
  __syncthreads();
  const Record rc = s_rc;
  if (rc.draw) {                                   // all accepted: the bonus token
    filtered_draw<DT, kVec>(A, b, rc, kDrawWaves);
    return;
  }
  if (!rc.pending) return;
  const int a = rc.a;
  const float c = rc.c;
  const float ip = 1.f / rc.Sp, iq = 1.f / rc.Sq;
  const Req req = request(A, b);
  const char* rowp = row_ptr(A, req, a);
  const char* rowq = row_ptr(A, req, A.R + a);
  // chunks wave, wave + kDrawWaves, ...: two at a time, all four row loads in flight
  for (int ch0 = wave; ch0 < A.n_chunk; ch0 += 2 * kDrawWaves) {
    ChunkRaw rp[2], rq[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int ch = ch0 + g * kDrawWaves;
      const int64_t c0 = (int64_t)ch * kCE;
      if (ch >= A.n_chunk) break;
      if (kVec && ch < A.n_full) {
        issue_chunk<DT>(rowp, c0, rp[g]);
        issue_chunk<DT>(rowq, c0, rq[g]);
      } else {
        load_chunk_checked<DT, kVec>(rowp, c0, A.V, rp[g]);
        load_chunk_checked<DT, kVec>(rowq, c0, A.V, rq[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int ch = ch0 + g * kDrawWaves;
      const int64_t c0 = (int64_t)ch * kCE;
      if (ch >= A.n_chunk) break;
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < kLoadsPerLane; ++j)
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const float yp = raw_elem<DT>(rp[g], j, k), yq = raw_elem<DT>(rq[g], j, k);
          const float wp = yp >= rc.tp ? fast_exp2(fmaf(yp, c, -rc.Mp)) * ip : 0.f;
          const float wq = yq >= rc.tq ? fast_exp2(fmaf(yq, c, -rc.Mq)) * iq : 0.f;
          sm += fmaxf(wp - wq, 0.f);
        }
      sm = wave_sum_all(sm);
      if (lane == 0) s_part[ch] = sm;
    }
  }
  __syncthreads();
  if (wave != 0) return;                           // the draw is one wave's work
  int found;
  float t_in;
  const float Z = wave_locate(A.n_chunk, rc.u, [&](int sg) { return s_part[sg]; }, &found, &t_in);
  int y = -1;
  if (Z > 0.f && found >= 0) {
    const int64_t c0 = (int64_t)found * kCE;
    float xp[E], xq[E], w[E];
    load_lane_run<DT, kVec, E>(rowp, c0, A.V, xp);
    load_lane_run<DT, kVec, E>(rowq, c0, A.V, xq);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const float wp = xp[k] >= rc.tp ? fast_exp2(fmaf(xp[k], c, -rc.Mp)) * ip : 0.f;
      const float wq = xq[k] >= rc.tq ? fast_exp2(fmaf(xq[k], c, -rc.Mq)) * iq : 0.f;
      w[k] = fmaxf(wp - wq, 0.f);
    }
    y = wave_pick<E>(w, c0, t_in);
  }
  if (y < 0) {                                     // p'_a and q'_a agree everywhere: draw from p'_a
    Record d = rc;
    d.xe = -1;
    filtered_draw<DT, kVec>(A, b, d, 1);           // this wave alone
    return;
  }
  if (lane == 0) A.out_tokens[(int64_t)b * A.out_cols + a] = y;
}

// The workspace header's give-up count, copied to out (and cleared when
// reset is set) in stream order.
__global__ void sv_errors_kernel(unsigned* err, uint32_t* out, int reset) {
  if (threadIdx.x == 0) {
    *out = reset ? __hip_atomic_exchange(err, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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

// Scratch of spec_verify_sample_noalloc, for callers that cannot allocate:
// the workspace of one call lives in this array (every device the library
// runs on holds its own copy until the process ends). Host code never uses
// its name as an address: each device's address comes from
// hipGetSymbolAddress (see scratch_on_current_device).
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// ================================================================ host ===
namespace {

using namespace sv;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t part, wpart, gath, rec, res, unif, alive, rf, fpart, tz, total;
  int64_t nch;     // chunks per row of the smaller (fp32) chunk: a bound for both dtypes
};

// Workspace: [header: the give-up count][counters: 4 * SV_MAX_BATCH]
//            [chunk partials][workgroup
//            partials][gathered logits][records][residual partials]
//            [uniforms][alive flags][row cuts][kept weight per chunk]
//            [tagged slots of one-launch calls]
Layout layout(int64_t B, int64_t rows, int64_t V) {
  const int64_t ce = Chunk<kF32>::kElems;          // the smaller chunk: a bound for both dtypes
  const int64_t nch = (V + ce - 1) / ce;
  Layout L;
  L.nch = nch;
  L.part = align_up(kHeaderBytes + kCounterBytes, 256);
  L.wpart = align_up(L.part + (size_t)(B * rows * nch) * sizeof(float2), 256);
  L.gath = align_up(L.wpart + (size_t)(B * rows * nch) * sizeof(float2), 256);   // wpr <= nch
  L.rec = align_up(L.gath + (size_t)(B * rows) * sizeof(float), 256);
  L.res = align_up(L.rec + (size_t)B * sizeof(Record), 256);
  L.unif = align_up(L.res + (size_t)(B * nch) * sizeof(float), 256);
  L.alive = align_up(L.unif + (size_t)(B * rows) * sizeof(float2), 256);   // R <= rows
  L.rf = align_up(L.alive + (size_t)B * sizeof(int), 256);
  L.fpart = align_up(L.rf + (size_t)(B * rows) * sizeof(RowFilter), 256);
  L.tz = align_up(L.fpart + (size_t)(B * rows * nch) * sizeof(float), 256);
  // tagged slots of one-launch calls: partials [2 words each], gathered
  // logits, uniforms [2 words each] (R <= rows, wpr <= nch)
  L.total = align_up(L.tz + (size_t)(B * rows * (2 * nch + 1 + 2)) * sizeof(uint64_t), 256);
  return L;
}

int elem_bytes(int dtype) { return dtype == SV_DTYPE_BF16 ? 2 : 4; }

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

// Chunks per workgroup: about 8192 workgroups, so the launch fills the chip
// in several whole rounds of resident workgroups (fewer, longer runs leave
// the last round a fraction full), at least one chunk per wave, and the runs
// of one row balanced (a 63-chunk row splits 11x5 + 8, not 12x5 + 3).
// SPECVERIFY_CHUNKS_PER_WG overrides the target run length (tuning).
// Small launches of long rows (one chunk per wave by that rule, and rows of
// at least 48 chunks) take four chunks per wave instead, so each wave's
// loads stay pipelined: B=32, K=5, V=128256 measured 18.4 us per call
// against 21.3 us with one chunk per wave.
int chunks_per_wg(int64_t rows_total, int n_chunk) {
  static const int env = [] {
    const char* e = getenv("SPECVERIFY_CHUNKS_PER_WG");
    return e ? atoi(e) : 0;
  }();
  int64_t target = env > 0 ? env : (rows_total * n_chunk + 8191) / 8192;
  if (env <= 0 && target <= kWaves && n_chunk >= 12 * kWaves) target = 4 * kWaves;
  if (target < kWaves) target = kWaves;
  if (target > kMaxChunksPerWg) target = kMaxChunksPerWg;
  const int64_t wpr = (n_chunk + target - 1) / target;
  return (int)((n_chunk + wpr - 1) / wpr);
}

// Early-exit rounds on long rows (at least 48 chunks): at least three
// chunks per wave, so each workgroup's loads stay pipelined (a round has
// few rows, and one-chunk runs left C3's round 0 at about half the
// streaming rate); still at least four workgroups per row. Shorter rows
// take one workgroup per row: B=64, K=3, V=32000 fp32 with draft logits
// measured 31.3 us per call against 41.1 with one chunk per wave (and
// 33.9 with whole rows in the second round only); C3's rows measured
// slower with longer runs (34.7 against 33.3 us at eight chunks per
// wave). Runs balanced as above.
int round_chunks_per_wg(int64_t rows_total, int n_chunk) {
  if (n_chunk < 12 * kWaves) return n_chunk;
  const int floor_len = 3 * kWaves;
  const int target = std::max(chunks_per_wg(rows_total, n_chunk), floor_len);
  const int wpr = (n_chunk + target - 1) / target;
  return (n_chunk + wpr - 1) / wpr;
}

// Test hooks, read at every call (unset in normal use):
//   SPECVERIFY_SPIN_LIMIT  polls before a one-launch tail gives up (default 2^20)
//   SPECVERIFY_DROP_TAGGED_REQUEST  a request whose row-pass workgroups skip
//                          their tagged stores in one-launch calls, so its tail
//                          gives up (exercises the give-up count)
//   SPECVERIFY_TAG         the tag of every one-launch call (hex; exercises tag
//                          repeats between calls)
int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return (e && *e) ? atoi(e) : dflt;
}
int spin_limit() {
  const int v = env_int("SPECVERIFY_SPIN_LIMIT", kSpinLimit);
  return v > 0 ? v : kSpinLimit;
}
int drop_request() { return env_int("SPECVERIFY_DROP_TAGGED_REQUEST", -1); }

// The first call that finds a device remembers it; until then every entry
// point asks the runtime (and clears the error a failed query leaves).
int device_status() {
  static std::atomic<int> found{0};
  if (found.load(std::memory_order_relaxed)) return SV_OK;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return SV_ERR_NO_DEVICE;
  }
  found.store(1, std::memory_order_relaxed);
  return SV_OK;
}

// One-launch sampling stores a run's words in one block (run_words): whole
// 128-byte lines when every row's blocks fit the 2 * nch words the layout
// gives a row, else packed (cpw + 1 words; wpr * (cpw + 1) <= 2 * n_chunk
// because runs are balanced: cpw <= n_chunk / wpr + 1, and wpr <= n_chunk / 4
// + 1 when cpw >= 4, else wpr = 1). Called again when cpw / wpr change.
void plan_run_blocks(Args& A, int64_t nch) {
  const int lines = (A.cpw + 1 + 15) / 16;
  if ((int64_t)A.wpr * 16 * lines <= 2 * nch) {
    A.run_block = 16 * lines;
    A.row_words = (int64_t)A.wpr * A.run_block;
  } else {
    A.run_block = A.cpw + 1;
    A.row_words = 2 * (int64_t)A.n_chunk;
  }
}

void fill_common(Args& A, const sv_logits* t, int B, int K, int V, int R, int rows, void* ws) {
  const int64_t es = elem_bytes(t->dtype);
  A.tgt = static_cast<const char*>(t->data);
  A.t_sb = t->stride_b * es;
  A.t_sk = t->stride_k * es;
  A.drf = nullptr; A.d_sb = 0; A.d_sk = 0;
  A.cu = nullptr; A.total_k = 0;
  A.mask = nullptr; A.mask_words = (V + 31) / 32;
  A.round = -1; A.round_hi = -1; A.round_rows = 0;
  A.B = B; A.K = K; A.V = V; A.R = R; A.rows = rows;
  const int ce = t->dtype == SV_DTYPE_BF16 ? Chunk<kBF16>::kElems : Chunk<kF32>::kElems;
  A.n_chunk = (V + ce - 1) / ce;
  A.n_full = V / ce;
  A.cpw = chunks_per_wg((int64_t)B * rows, A.n_chunk);
  A.wpr = (A.n_chunk + A.cpw - 1) / A.cpw;
  const Layout L = layout(B, rows, V);
  unsigned char* base = static_cast<unsigned char*>(ws);
  A.err = reinterpret_cast<unsigned*>(base);
  A.counters = reinterpret_cast<unsigned*>(base + kHeaderBytes);
  A.part = reinterpret_cast<float2*>(base + L.part);
  A.wpart = reinterpret_cast<float2*>(base + L.wpart);
  A.gath = reinterpret_cast<float*>(base + L.gath);
  A.rec = reinterpret_cast<Record*>(base + L.rec);
  A.res_part = reinterpret_cast<float*>(base + L.res);
  A.unif = reinterpret_cast<float2*>(base + L.unif);
  A.alive = reinterpret_cast<int*>(base + L.alive);
  A.rf = reinterpret_cast<RowFilter*>(base + L.rf);
  A.fpart = reinterpret_cast<float*>(base + L.fpart);
  A.tz_part = reinterpret_cast<uint64_t*>(base + L.tz);
  A.tz_gath = A.tz_part + 2 * (size_t)(B * rows * L.nch);
  A.tz_unif = A.tz_gath + (size_t)(B * rows);
  plan_run_blocks(A, L.nch);
  A.tag = 0;
  A.n_rowwg = 0;
  A.spin_limit = spin_limit();
  A.drop_req = drop_request();
  A.no_tail = 0;
  A.filtered = 0;
  A.top_k = nullptr;
  A.top_p = nullptr;
  A.out_p = nullptr; A.out_q = nullptr; A.out_aux = nullptr;
  A.temperature = nullptr; A.seeds = nullptr; A.offset = 0;
  A.n_nodes = 0;
  for (int i = 0; i < SV_MAX_TREE_NODES; ++i) { A.parent[i] = -1; A.depth[i] = 0; }
  A.dyn_parents = nullptr;
}

#define SV_LAUNCH(KERNEL, grid, st, A) \
  hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(kThreads), 0, st, A)

// Row pass over every (request, row, chunk run), then one tail wave per
// request, back to back on the caller's stream.
// A one-launch call (A.n_rowwg > 0): the row pass's workgroups and then one
// tail workgroup per request, in one grid.
template <int MODE, int DT, bool kVec, bool kMask>
void launch_pair(const Args& A, unsigned grid, hipStream_t st) {
  if constexpr (MODE != kExplicit) {              // draft logits: never one launch
    if (A.n_rowwg > 0) {
      SV_LAUNCH((sv_rows_kernel<MODE, DT, kVec, kMask, false, true>), grid + (unsigned)A.B, st, A);
      return;
    }
  }
  SV_LAUNCH((sv_rows_kernel<MODE, DT, kVec, kMask, false, false>), grid, st, A);
  if (A.no_tail) return;                           // the residual pass runs the rule
  hipLaunchKernelGGL((sv_tail_kernel<MODE, DT, kVec, kMask>), dim3((unsigned)A.B), dim3(64), 0, st, A);
}

template <int MODE, int DT>
void launch_rows_dt(const Args& A, bool vec, bool mask, unsigned grid, hipStream_t st) {
  if constexpr (MODE == kTree) {                   // trees take no bitmask
    if (vec) launch_pair<MODE, DT, true, false>(A, grid, st);
    else     launch_pair<MODE, DT, false, false>(A, grid, st);
  } else {
    if (vec) {
      if (mask) launch_pair<MODE, DT, true, true>(A, grid, st);
      else      launch_pair<MODE, DT, true, false>(A, grid, st);
    } else {
      if (mask) launch_pair<MODE, DT, false, true>(A, grid, st);
      else      launch_pair<MODE, DT, false, false>(A, grid, st);
    }
  }
}

template <int MODE>
void launch_rows(const Args& A, int dtype, bool vec, unsigned grid, hipStream_t st) {
  const bool mask = A.mask != nullptr;
  if (dtype == SV_DTYPE_BF16) launch_rows_dt<MODE, kBF16>(A, vec, mask, grid, st);
  else                        launch_rows_dt<MODE, kF32>(A, vec, mask, grid, st);
}

// decide: the residual pass runs the rule itself (no tail launch before it).
template <int DT, bool kDecide>
void launch_residual_dd(const Args& A, bool vec, unsigned grid, hipStream_t st) {
  const bool mask = A.mask != nullptr, filt = A.filtered != 0;
  if (vec) {
    if (filt)      SV_LAUNCH((sv_residual_kernel<DT, true, false, true, kDecide>), grid, st, A);
    else if (mask) SV_LAUNCH((sv_residual_kernel<DT, true, true, false, kDecide>), grid, st, A);
    else           SV_LAUNCH((sv_residual_kernel<DT, true, false, false, kDecide>), grid, st, A);
  } else {
    if (filt)      SV_LAUNCH((sv_residual_kernel<DT, false, false, true, kDecide>), grid, st, A);
    else if (mask) SV_LAUNCH((sv_residual_kernel<DT, false, true, false, kDecide>), grid, st, A);
    else           SV_LAUNCH((sv_residual_kernel<DT, false, false, false, kDecide>), grid, st, A);
  }
}

template <int DT>
void launch_residual_dt(const Args& A, bool vec, unsigned grid, hipStream_t st, bool decide) {
  if constexpr (DT == kF32) {                      // bf16 chunks would not fit its registers
    if (decide && A.filtered && A.n_chunk <= kRes1Chunks) {   // one workgroup per request
      const dim3 reqs((unsigned)A.B), wg(kDrawThreads);
      if (vec) hipLaunchKernelGGL((sv_fresidual_kernel<DT, true>), reqs, wg, 0, st, A);
      else     hipLaunchKernelGGL((sv_fresidual_kernel<DT, false>), reqs, wg, 0, st, A);
      return;
    }
  }
  if (decide) {
    launch_residual_dd<DT, true>(A, vec, grid, st);
  } else {
    launch_residual_dd<DT, false>(A, vec, grid, st);
  }
}

// Filtered verification: per row the cut and kept mass (bf16: the one-pass
// histogram kernel; fp32 rows of at most kRCap logits: the register-resident
// select; longer fp32 rows: the row pass, then the select pass), one
// workgroup per row; then the filtered rule and the draw, one workgroup per
// request. With draft logits the residual pass that follows runs the rule
// itself.
template <int MODE, int DT>
void launch_filtered_dt(const Args& A, bool vec, unsigned grid, hipStream_t st) {
  const dim3 rows((unsigned)((int64_t)A.B * A.rows)), reqs((unsigned)A.B), wg(kThreads), dwg(kDrawThreads);
  if constexpr (DT == kBF16) {
    if (vec) hipLaunchKernelGGL((sv_hselect_kernel<MODE, true>), rows, wg, 0, st, A);
    else     hipLaunchKernelGGL((sv_hselect_kernel<MODE, false>), rows, wg, 0, st, A);
  } else if (A.V <= kRCap) {
    const dim3 rwg(kRThreads);
    if (vec) hipLaunchKernelGGL((sv_rselect_kernel<MODE, true>), rows, rwg, 0, st, A);
    else     hipLaunchKernelGGL((sv_rselect_kernel<MODE, false>), rows, rwg, 0, st, A);
  } else {
    if (vec) {
      SV_LAUNCH((sv_rows_kernel<MODE, DT, true, false, false, false>), grid, st, A);
      hipLaunchKernelGGL((sv_select_kernel<MODE, DT, true>), rows, wg, 0, st, A);
    } else {
      SV_LAUNCH((sv_rows_kernel<MODE, DT, false, false, false, false>), grid, st, A);
      hipLaunchKernelGGL((sv_select_kernel<MODE, DT, false>), rows, wg, 0, st, A);
    }
  }
  if constexpr (MODE != kExplicit) {
    if (vec) hipLaunchKernelGGL((sv_ftail_kernel<MODE, DT, true>), reqs, dwg, 0, st, A);
    else     hipLaunchKernelGGL((sv_ftail_kernel<MODE, DT, false>), reqs, dwg, 0, st, A);
  }
}

template <int MODE>
void launch_filtered(const Args& A, int dtype, bool vec, unsigned grid, hipStream_t st) {
  if (dtype == SV_DTYPE_BF16) launch_filtered_dt<MODE, kBF16>(A, vec, grid, st);
  else                        launch_filtered_dt<MODE, kF32>(A, vec, grid, st);
}

void launch_residual(const Args& A, int dtype, bool vec, unsigned grid, hipStream_t st,
                     bool decide = false) {
  if (dtype == SV_DTYPE_BF16) launch_residual_dt<kBF16>(A, vec, grid, st, decide);
  else                        launch_residual_dt<kF32>(A, vec, grid, st, decide);
}

// One early-exit round: the row pass over this round's rows, which ends in
// the per-request decision.
template <int MODE>
void launch_round(const Args& A, int dtype, bool vec, unsigned grid, hipStream_t st) {
  if (dtype == SV_DTYPE_BF16) {
    if (vec) SV_LAUNCH((sv_rows_kernel<MODE, kBF16, true, false, true, false>), grid, st, A);
    else     SV_LAUNCH((sv_rows_kernel<MODE, kBF16, false, false, true, false>), grid, st, A);
  } else {
    if (vec) SV_LAUNCH((sv_rows_kernel<MODE, kF32, true, false, true, false>), grid, st, A);
    else     SV_LAUNCH((sv_rows_kernel<MODE, kF32, false, false, true, false>), grid, st, A);
  }
}

// One-launch calls. Every call takes a fresh tag: a negative-NaN pattern
// (0xFF800001 ... 0xFFFFFFFF) from a per-process counter that starts at a
// clock-derived value, so a library loaded again does not repeat the tags
// still in a workspace. Tail workgroups may be resident before the last
// row-pass workgroups, so the batch is capped (1024 tail workgroups leave
// most of every CU to the row pass). SPECVERIFY_ONE_LAUNCH=0 in the
// environment at the time of a call selects the two-launch path (the same
// results up to fp32 rounding order; timing comparisons and tests).
constexpr int kFusedMaxBatch = 1024;

uint32_t next_tag() {
  static std::atomic<uint32_t> counter{
      (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count()};
  uint32_t v = counter.fetch_add(1u, std::memory_order_relaxed);
  if (const char* e = getenv("SPECVERIFY_TAG")) v = (uint32_t)strtoul(e, nullptr, 16) - 1u;   // test hook
  return 0xFF800000u | (1u + v % 0x7FFFFFu);
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; the first lookup also zero-
// fills the array on `st` (a fill kernel), so the counters and tagged words
// start at zero. Every later call leaves them zero again.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_on_current_device(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SV_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SV_ERR_HIP;
    }
    hipLaunchKernelGGL(sv_zero_kernel, dim3(4096), dim3(kThreads), 0, st,
                       static_cast<unsigned char*>(p), kScratchBytes);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}

bool one_launch_enabled() {
  const char* e = getenv("SPECVERIFY_ONE_LAUNCH");
  return !(e && e[0] == '0');
}

// Whether the tail's loads fit: sampling, every chunk partial of the
// request in kFusedQ loads per lane; argmax, the workgroup partials in
// wstage_issue's grouped layout.
bool one_launch_fits(const Args& A, int mode) {
  if (!one_launch_enabled() || A.B > kFusedMaxBatch) return false;
  if (mode == kOneHot || mode == kExplicit) return A.rows * ((A.n_chunk + 63) / 64) <= kFusedQ;
  int G = 1;
  while (G < A.wpr) G <<= 1;
  if (G > 64) return false;
  return (A.rows + 64 / G - 1) / (64 / G) <= 8;
}

// Marks A as a one-launch call when it fits. Calls with draft logits keep
// two launches: a residual pass follows anyway and runs the rule itself,
// which measured faster at every size (B=64, K=3, V=32000: 19.8 against
// 28.5 us in one launch; B=1, K=1, V=1000: 8.9 against 10.4 us).
void plan_one_launch(Args& A, int mode, int64_t row_wgs) {
  if (mode == kExplicit) return;
  if (!one_launch_fits(A, mode) || row_wgs + A.B > (int64_t)(UINT32_MAX / kThreads)) return;
  A.n_rowwg = (int)row_wgs;
  A.tag = next_tag();
}

// Greedy and tree row passes (an argmax per chunk, no exponentials): when
// the general rule gives one chunk per wave and rows hold at least 24
// chunks, runs take three per wave (the 31-node tree of B=32, V=32000 fp32
// measured 27.1 us per call against 28.3 us); wpr and cpw are recomputed.
void argmax_runs(Args& A) {
  if (getenv("SPECVERIFY_CHUNKS_PER_WG")) return;  // a tuning override stands as given
  if (A.cpw > kWaves || A.n_chunk < 6 * kWaves) return;
  const int wpr = (A.n_chunk + 3 * kWaves - 1) / (3 * kWaves);
  A.cpw = (A.n_chunk + wpr - 1) / wpr;
  A.wpr = (A.n_chunk + A.cpw - 1) / A.cpw;
}

// A dispatch counts work-items in 32 bits per dimension.
int check_grid(int64_t wgs) {
  return (wgs >= 1 && wgs <= (int64_t)(UINT32_MAX / kThreads)) ? SV_OK : SV_ERR_SHAPE;
}

int hip_status() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP; }

// Host checks of a sampling call's arguments (everything but the workspace).
int check_sample_args(const sv_logits* target, const sv_logits* draft, const int32_t* cu,
                      int32_t total_k, const int32_t* draft_tokens, const float* temperature,
                      const uint64_t* seeds, int32_t B, int32_t K, int32_t V,
                      const int32_t* out_tokens, const int32_t* out_accept_len) {
  int st = check_desc(target);
  if (st) return st;
  if (draft && (st = check_desc(draft))) return st;
  if (!temperature || !seeds || !out_tokens || !out_accept_len) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_DRAFT || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if ((cu ? total_k > 0 : K > 0) && !draft_tokens) return SV_ERR_NULL;
  if (draft && draft->dtype != target->dtype) return SV_ERR_DTYPE;
  return SV_OK;
}

// Sampling, dense (cu null: [B, K + 1] rows by the two strides) or ragged
// (cu [B + 1] device prefix sums, packed rows by stride_k, stride_b unused).
int sample_impl(const sv_logits* target, const sv_logits* draft, const int32_t* cu, int32_t total_k,
                const uint32_t* mask, bool lazy, const int32_t* top_k, const float* top_p,
                bool filtered, const int32_t* draft_tokens, const float* temperature,
                const uint64_t* seeds, uint64_t offset,
                int32_t B, int32_t K, int32_t V,
                int32_t* out_tokens, int32_t* out_accept_len,
                float* out_p_draft, float* out_q_draft,
                void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_sample_args(target, draft, cu, total_k, draft_tokens, temperature, seeds, B, K, V,
                             out_tokens, out_accept_len);
  if (st) return st;
  if (!workspace) return SV_ERR_WORKSPACE;
  const bool explicit_q = draft != nullptr && K > 0;
  const int R = K + 1;
  const int rows = R + (explicit_q ? K : 0);
  if (workspace_bytes < layout(B, rows, V).total) return SV_ERR_WORKSPACE;
  if ((st = device_status())) return st;

  Args A;
  fill_common(A, target, B, K, V, R, rows, workspace);
  if (explicit_q) {
    const int64_t es = elem_bytes(draft->dtype);
    A.drf = static_cast<const char*>(draft->data);
    A.d_sb = draft->stride_b * es;
    A.d_sk = draft->stride_k * es;
  }
  A.tokens = draft_tokens;
  A.cu = cu;
  A.total_k = total_k;
  A.mask = mask;
  A.temperature = temperature;
  A.seeds = seeds;
  A.offset = offset;
  A.out_cols = K + 1;
  A.out_tokens = out_tokens;
  A.out_len = out_accept_len;
  A.out_p = out_p_draft;
  A.out_q = out_q_draft;
  const bool vec = aligned16(target) && (!explicit_q || aligned16(draft));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (filtered) {
    A.filtered = 1;
    A.top_k = top_k;
    A.top_p = top_p;
    const int64_t wgs = (int64_t)B * rows * A.wpr;
    if ((st = check_grid(wgs))) return st;
    if (explicit_q) launch_filtered<kExplicit>(A, target->dtype, vec, (unsigned)wgs, s);
    else            launch_filtered<kOneHot>(A, target->dtype, vec, (unsigned)wgs, s);
    if ((st = hip_status())) return st;
    if (explicit_q) {                              // the residual pass runs the filtered rule
      Args A2 = A;
      A2.cpw = chunks_per_wg(B, A.n_chunk);
      A2.wpr = (A.n_chunk + A2.cpw - 1) / A2.cpw;
      launch_residual(A2, target->dtype, vec, (unsigned)((int64_t)B * A2.wpr), s, true);
    }
    return hip_status();
  }
  if (lazy) {                                      // early-exit rounds
    // windows of positions [0], then [1, K]
    for (int lo = 0, w = 1; lo <= K; lo += w, w = K) {
      const int hi = std::min(lo + w - 1, (int)K);
      Args Ai = A;
      Ai.round = lo;
      Ai.round_hi = hi;
      Ai.round_rows = (hi - lo + 1) + (explicit_q ? std::max(0, std::min(hi, K - 1) - lo + 1) : 0);
      Ai.cpw = round_chunks_per_wg((int64_t)B * Ai.round_rows, A.n_chunk);
      Ai.wpr = (A.n_chunk + Ai.cpw - 1) / Ai.cpw;
      const int64_t g = (int64_t)B * Ai.round_rows * Ai.wpr;
      if ((st = check_grid(g))) return st;
      if (explicit_q) launch_round<kExplicit>(Ai, target->dtype, vec, (unsigned)g, s);
      else            launch_round<kOneHot>(Ai, target->dtype, vec, (unsigned)g, s);
      if ((st = hip_status())) return st;
    }
    if (explicit_q) {
      Args A2 = A;
      A2.cpw = chunks_per_wg(B, A.n_chunk);
      A2.wpr = (A.n_chunk + A2.cpw - 1) / A2.cpw;
      launch_residual(A2, target->dtype, vec, (unsigned)((int64_t)B * A2.wpr), s);
    }
    return hip_status();
  }
  const int64_t wgs = (int64_t)B * rows * A.wpr;
  if ((st = check_grid(wgs))) return st;
  plan_one_launch(A, explicit_q ? kExplicit : kOneHot, wgs);
  if (explicit_q) {
    // the row pass, then the residual pass, whose workgroups run the rule
    // themselves (no tail launch between)
    const bool decide = A.n_rowwg == 0;
    A.no_tail = decide ? 1 : 0;
    launch_rows<kExplicit>(A, target->dtype, vec, (unsigned)wgs, s);
    if ((st = hip_status())) return st;
    // the residual pass streams one stop row pair per request
    Args A2 = A;
    A2.n_rowwg = 0;
    A2.cpw = chunks_per_wg(B, A.n_chunk);
    A2.wpr = (A.n_chunk + A2.cpw - 1) / A2.cpw;
    launch_residual(A2, target->dtype, vec, (unsigned)((int64_t)B * A2.wpr), s, decide);
  } else {
    launch_rows<kOneHot>(A, target->dtype, vec, (unsigned)wgs, s);
  }
  return hip_status();
}

// Greedy, dense or ragged (as sample_impl).
int greedy_impl(const sv_logits* target, const int32_t* cu, int32_t total_k, const uint32_t* mask,
                const int32_t* draft_tokens, int32_t B, int32_t K, int32_t V,
                int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(target);
  if (st) return st;
  if (!out_tokens || !out_accept_len) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || K < 0 || K > SV_MAX_DRAFT || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if ((cu ? total_k > 0 : K > 0) && !draft_tokens) return SV_ERR_NULL;
  if (!workspace) return SV_ERR_WORKSPACE;
  const int R = K + 1;
  if (workspace_bytes < layout(B, R, V).total) return SV_ERR_WORKSPACE;
  if ((st = device_status())) return st;
  Args A;
  fill_common(A, target, B, K, V, R, R, workspace);
  A.tokens = draft_tokens;
  A.cu = cu;
  A.total_k = total_k;
  A.mask = mask;
  A.out_cols = K + 1;
  A.out_tokens = out_tokens;
  A.out_len = out_accept_len;
  A.out_aux = out_argmax;
  argmax_runs(A);
  const int64_t wgs = (int64_t)B * R * A.wpr;
  if ((st = check_grid(wgs))) return st;
  plan_one_launch(A, kGreedy, wgs);
  launch_rows<kGreedy>(A, target->dtype, aligned16(target), (unsigned)wgs,
                       static_cast<hipStream_t>(stream));
  return hip_status();
}

}  // namespace

namespace {

// Tree verification, static (host parents, checked here) or dynamic (one
// parent row per request on the device, checked by the tail).
int tree_impl(const sv_logits* target, const int32_t* node_tokens, const int32_t* parents, bool dynamic,
              int32_t N, int32_t B, int32_t V, int32_t* out_tokens, int32_t* out_accept_len,
              int32_t* out_best_node, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(target);
  if (st) return st;
  if (!node_tokens || !parents || !out_tokens || !out_accept_len) return SV_ERR_NULL;
  if (B < 1 || B > SV_MAX_BATCH || V < 1 || V > SV_MAX_VOCAB || N < 2 || N > SV_MAX_TREE_NODES)
    return SV_ERR_SHAPE;
  if (!dynamic) {
    if (parents[0] != -1) return SV_ERR_TREE;
    for (int n = 1; n < N; ++n)
      if (parents[n] < 0 || parents[n] >= n) return SV_ERR_TREE;
  }
  if (!workspace) return SV_ERR_WORKSPACE;
  if (workspace_bytes < layout(B, N, V).total) return SV_ERR_WORKSPACE;
  if ((st = device_status())) return st;
  Args A;
  fill_common(A, target, B, 0, V, N, N, workspace);
  A.tokens = node_tokens;
  A.out_cols = N;
  A.out_tokens = out_tokens;
  A.out_len = out_accept_len;
  A.out_aux = out_best_node;
  A.n_nodes = N;
  if (dynamic) {
    A.dyn_parents = parents;
  } else {
    for (int n = 0; n < N; ++n) {
      A.parent[n] = (int8_t)parents[n];
      A.depth[n] = (int8_t)(n == 0 ? 0 : A.depth[parents[n]] + 1);   // parents[n] < n
    }
  }
  argmax_runs(A);
  const int64_t wgs = (int64_t)B * N * A.wpr;
  if ((st = check_grid(wgs))) return st;
  plan_one_launch(A, kTree, wgs);
  launch_rows<kTree>(A, target->dtype, aligned16(target), (unsigned)wgs,
                     static_cast<hipStream_t>(stream));
  return hip_status();
}

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
  if (const int st = device_status()) return st;
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
  return sample_impl(target, draft, nullptr, 0, nullptr, false, nullptr, nullptr, false, draft_tokens,
                     temperature, seeds, offset, B, K, V, out_tokens, out_accept_len, out_p_draft,
                     out_q_draft, workspace, workspace_bytes, stream);
}

int spec_verify_sample_noalloc(const sv_logits* target, const sv_logits* draft,
                               const int32_t* draft_tokens, const float* temperature,
                               const uint64_t* seeds, uint64_t offset,
                               int32_t B, int32_t K, int32_t V,
                               int32_t* out_tokens, int32_t* out_accept_len,
                               float* out_p_draft, float* out_q_draft, void* stream) {
  int st = check_sample_args(target, draft, nullptr, 0, draft_tokens, temperature, seeds, B, K, V,
                             out_tokens, out_accept_len);
  if (st) return st;
  const int rows = K + 1 + ((draft && K > 0) ? K : 0);
  if (layout(B, rows, V).total > kScratchBytes) return SV_ERR_SCRATCH;
  if ((st = device_status())) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = scratch_on_current_device(s, &ws))) return st;
  return sample_impl(target, draft, nullptr, 0, nullptr, false, nullptr, nullptr, false, draft_tokens,
                     temperature, seeds, offset, B, K, V, out_tokens, out_accept_len, out_p_draft,
                     out_q_draft, ws, kScratchBytes, stream);
}

int spec_verify_sample_lazy(const sv_logits* target, const sv_logits* draft,
                            const int32_t* draft_tokens, const float* temperature,
                            const uint64_t* seeds, uint64_t offset,
                            int32_t B, int32_t K, int32_t V,
                            int32_t* out_tokens, int32_t* out_accept_len,
                            float* out_p_draft, float* out_q_draft,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return sample_impl(target, draft, nullptr, 0, nullptr, true, nullptr, nullptr, false, draft_tokens,
                     temperature, seeds, offset, B, K, V, out_tokens, out_accept_len, out_p_draft,
                     out_q_draft, workspace, workspace_bytes, stream);
}

int spec_verify_sample_filtered(const sv_logits* target, const sv_logits* draft,
                                const int32_t* draft_tokens, const float* temperature,
                                const int32_t* top_k, const float* top_p,
                                const uint64_t* seeds, uint64_t offset,
                                int32_t B, int32_t K, int32_t V,
                                int32_t* out_tokens, int32_t* out_accept_len,
                                float* out_p_draft, float* out_q_draft,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return sample_impl(target, draft, nullptr, 0, nullptr, false, top_k, top_p, true, draft_tokens,
                     temperature, seeds, offset, B, K, V, out_tokens, out_accept_len, out_p_draft,
                     out_q_draft, workspace, workspace_bytes, stream);
}

int spec_verify_sample_masked(const sv_logits* target, const sv_logits* draft,
                              const int32_t* draft_tokens, const uint32_t* bitmask,
                              const float* temperature, const uint64_t* seeds, uint64_t offset,
                              int32_t B, int32_t K, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_p_draft, float* out_q_draft,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!bitmask) return SV_ERR_NULL;
  return sample_impl(target, draft, nullptr, 0, bitmask, false, nullptr, nullptr, false, draft_tokens,
                     temperature, seeds, offset, B, K, V, out_tokens, out_accept_len, out_p_draft,
                     out_q_draft, workspace, workspace_bytes, stream);
}

int spec_verify_sample_ragged(const sv_logits* target, const sv_logits* draft,
                              const int32_t* cu_draft, int32_t total_k,
                              const int32_t* draft_tokens, const float* temperature,
                              const uint64_t* seeds, uint64_t offset,
                              int32_t B, int32_t K_max, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_p_draft, float* out_q_draft,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_draft || !target) return SV_ERR_NULL;
  if (total_k < 0) return SV_ERR_SHAPE;
  sv_logits t = *target, d = draft ? *draft : sv_logits{};
  t.stride_b = 0;                                   // packed rows: stride_k only
  d.stride_b = 0;
  return sample_impl(&t, draft ? &d : nullptr, cu_draft, total_k, nullptr, false, nullptr, nullptr,
                     false, draft_tokens, temperature, seeds, offset, B, K_max, V, out_tokens,
                     out_accept_len, out_p_draft, out_q_draft, workspace, workspace_bytes, stream);
}

int spec_verify_greedy(const sv_logits* target, const int32_t* draft_tokens,
                       int32_t B, int32_t K, int32_t V,
                       int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return greedy_impl(target, nullptr, 0, nullptr, draft_tokens, B, K, V, out_tokens, out_accept_len,
                     out_argmax, workspace, workspace_bytes, stream);
}

int spec_verify_greedy_masked(const sv_logits* target, const int32_t* draft_tokens,
                              const uint32_t* bitmask, int32_t B, int32_t K, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!bitmask) return SV_ERR_NULL;
  return greedy_impl(target, nullptr, 0, bitmask, draft_tokens, B, K, V, out_tokens, out_accept_len,
                     out_argmax, workspace, workspace_bytes, stream);
}

int spec_verify_greedy_ragged(const sv_logits* target, const int32_t* cu_draft, int32_t total_k,
                              const int32_t* draft_tokens, int32_t B, int32_t K_max, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_draft || !target) return SV_ERR_NULL;
  if (total_k < 0) return SV_ERR_SHAPE;
  sv_logits t = *target;
  t.stride_b = 0;
  return greedy_impl(&t, cu_draft, total_k, nullptr, draft_tokens, B, K_max, V, out_tokens,
                     out_accept_len, out_argmax, workspace, workspace_bytes, stream);
}

int spec_verify_tree(const sv_logits* target, const int32_t* node_tokens,
                     const int32_t* parents, int32_t N, int32_t B, int32_t V,
                     int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_best_node,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return tree_impl(target, node_tokens, parents, false, N, B, V, out_tokens, out_accept_len, out_best_node,
                   workspace, workspace_bytes, stream);
}

int spec_verify_tree_dynamic(const sv_logits* target, const int32_t* node_tokens,
                             const int32_t* parents, int32_t N, int32_t B, int32_t V,
                             int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_best_node,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return tree_impl(target, node_tokens, parents, true, N, B, V, out_tokens, out_accept_len, out_best_node,
                   workspace, workspace_bytes, stream);
}

int spec_verify_workspace_errors(void* workspace, size_t workspace_bytes, uint32_t* out_count,
                                 int32_t reset, void* stream) {
  if (!workspace || !out_count) return SV_ERR_NULL;
  if (workspace_bytes < kHeaderBytes) return SV_ERR_WORKSPACE;
  if (const int st = device_status()) return st;
  hipLaunchKernelGGL(sv_errors_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<unsigned*>(workspace), out_count, reset);
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
    case SV_ERR_NO_DEVICE: return "no HIP device visible";
    case SV_ERR_SCRATCH: return "the call needs more than the 16 MiB of spec_verify_sample_noalloc's scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
