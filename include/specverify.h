/*
 * specverify.h — C ABI of the MI355X (gfx950) speculative-decoding verifier.
 *
 * One target forward over K+1 positions yields the logits of K+1 target
 * distributions per request; these entry points decide which of the K draft
 * tokens are accepted and produce the one extra token (replacement or bonus)
 * of the step ("【大模型基础设施工程】15：推测解码与 MTP", juejin: §1.2 and
 * §2.1). Requests are verified in parallel, one batch per call (FastDeploy
 * "投机解码", "高效投机解码框架设计": parallel sampling + verification per
 * batch sample).
 *
 * Conventions shared by every entry point
 *  - Every pointer is a DEVICE pointer unless its comment says [host].
 *  - Logits are row-major with the vocabulary innermost (stride 1) and
 *    described by sv_logits; strides are in ELEMENTS and may be 0
 *    (broadcast). Rows whose address and strides are 16-byte aligned take
 *    the 128-bit load path, others a scalar path with identical results.
 *  - The caller owns every buffer. The library allocates nothing, never
 *    synchronises and launches only on `stream` (a hipStream_t; NULL = the
 *    default stream). Results are ready when the stream reaches them. Its
 *    only state is a per-process counter that numbers one-launch calls
 *    (below) and a flag that remembers that a device was found.
 *  - Argument errors are detected on the host before anything is launched
 *    and returned as a negative status; nothing is written then. With
 *    valid arguments and no HIP device visible a call returns
 *    SV_ERR_NO_DEVICE. Device-resident values are not checked on the host;
 *    their handling is stated per entry point.
 *  - Workspace: size from spec_verify_workspace_size(), zero-filled ONCE by
 *    spec_verify_workspace_init() (or any zero fill) before its first use.
 *    Every call leaves the workspace's counter words zero again, so it can
 *    be reused by any later call that fits; it must not be shared by calls
 *    that may run concurrently (different streams). Calls that run the
 *    row pass and the per-request rule in one launch hand results over
 *    through workspace words tagged with the call's number (a per-process
 *    counter with period 2^23 - 1); the rule's workgroups clear every such
 *    word once they have read it, so after each call the tagged words are
 *    zero again and a word of an earlier call can never be taken for a
 *    later call's, even when their numbers repeat. Setting
 *    SPECVERIFY_ONE_LAUNCH=0 in the environment makes every call use two
 *    launches (the same results up to fp32 summation order). The wait for
 *    those words is bounded (2^20 polls, each at least one trip to memory);
 *    a request whose words never arrive, which a working device does not
 *    produce, is refused (accept length 0, tokens -1) rather than left
 *    hanging, and the event is counted in the workspace header, readable
 *    with spec_verify_workspace_errors(); a workspace with a nonzero count
 *    may hold stale words and should be zero-filled again.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SV_OK             0
#define SV_ERR_NULL      -1   /* a required pointer is NULL */
#define SV_ERR_SHAPE     -2   /* B, K, N or V out of range */
#define SV_ERR_DTYPE     -3   /* unknown dtype or reserved field not 0 */
#define SV_ERR_STRIDE    -4   /* negative stride */
#define SV_ERR_WORKSPACE -5   /* workspace NULL or smaller than required */
#define SV_ERR_TREE      -6   /* malformed parent array */
#define SV_ERR_HIP       -7   /* a HIP launch failed (hipGetLastError) */
#define SV_ERR_NO_DEVICE -8   /* no HIP device is visible */
#define SV_ERR_SCRATCH   -9   /* a no-allocation call needs more than its scratch holds */

/* logits element types */
#define SV_DTYPE_F32  0
#define SV_DTYPE_BF16 1

/* operation ids for spec_verify_workspace_size */
#define SV_OP_SAMPLE 0
#define SV_OP_GREEDY 1
#define SV_OP_TREE   2

/* limits */
#define SV_MAX_BATCH      65536
#define SV_MAX_DRAFT      32          /* K */
#define SV_MAX_TREE_NODES 64          /* N, root included */
#define SV_MAX_VOCAB      (1 << 30)

/* A [B, rows, V] logits tensor: element (b, r, v) is at
 * data + (b * stride_b + r * stride_k + v) * sizeof(element). */
typedef struct sv_logits {
  const void* data;    /* device pointer to element (0, 0, 0) */
  int32_t dtype;       /* SV_DTYPE_F32 or SV_DTYPE_BF16 */
  int32_t reserved;    /* must be 0 */
  int64_t stride_b;    /* elements between requests, >= 0 */
  int64_t stride_k;    /* elements between positions (rows), >= 0 */
} sv_logits;

/*
 * Bytes of workspace needed by one call of `op` with batch B, K drafts
 * (SV_OP_TREE: N nodes) and vocabulary V; `has_draft` is 1 when
 * spec_verify_sample gets draft logits. The value is valid for either
 * logits dtype. Returns 0 for arguments out of range.
 */
size_t spec_verify_workspace_size(int32_t op, int32_t B, int32_t K_or_N, int32_t V,
                                  int32_t has_draft);

/* Zero-fill `workspace_bytes` bytes of a workspace on `stream` (a fill
 * kernel, no memset node). SV_ERR_NULL for a NULL workspace. */
int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Health of a workspace (not an operation of the pages: it reports on the
 * library's own one-launch hand-off). Writes to out_count (a DEVICE
 * uint32) the number of requests, over every call since the workspace was
 * zero-filled (or since the last reset), whose rule gave up waiting for
 * the row pass's words and refused the request; with reset != 0 the count
 * is cleared at the same time. Runs in stream order: the value covers the
 * calls enqueued before it. A working device never gives up, so a nonzero
 * count means the refusals it counts were not the caller's doing and the
 * workspace should be zero-filled again (spec_verify_workspace_init).
 * SV_ERR_NULL for a NULL workspace or out_count, SV_ERR_WORKSPACE when
 * workspace_bytes is below the 256-byte header.
 */
int spec_verify_workspace_errors(void* workspace, size_t workspace_bytes, uint32_t* out_count,
                                 int32_t reset, void* stream);

/*
 * Stochastic verification ("推测解码与 MTP" §2.1; exactness: the
 * correctness subsection under §2).
 *
 * For request b with temperature T = temperature[b]:
 *   p_i = softmax(target[b, i, :] / T), i = 0..K        (K+1 rows)
 *   q_i = softmax(draft[b, i, :] / T), i = 0..K-1; when draft == NULL q_i is
 *         one-hot at draft_tokens[b, i] (n-gram / MTP drafts).
 *   Draft x_i = draft_tokens[b, i] is accepted when u_i * q_i(x_i) < p_i(x_i),
 *   i.e. with probability min(1, p_i(x_i) / q_i(x_i)); the scan stops at
 *   the first rejection a, where one token is drawn from the normalised
 *   residual max(0, p_a - q_a) (p_a if that has no mass); if all K are
 *   accepted the token is drawn from p_K. With draft logits the test is
 *   evaluated as log2 u + log2 q_i(x_i) < log2 p_i(x_i) (the same event;
 *   it stays exact where both probabilities underflow fp32). Draws are
 *   inverse-CDF: the
 *   smallest token whose running sum exceeds u times the total.
 *   The two uniforms of (b, i) are the top 24 bits of words 0 and 1 of
 *   Philox4x64-10 (Salmon et al., SC'11) with counter (i, b, offset, 0) and
 *   key (seeds[b], 0); the same (seeds, offset) replays a call exactly.
 *
 * target        [B, K+1, V] logits (fp32 or bf16)
 * draft         [host] NULL, or [B, >=K, V] logits (only rows 0..K-1 read)
 * draft_tokens  [B, K] int32, row-major; may be NULL when K == 0
 * temperature   [B] float, > 0
 * seeds         [B] uint64
 * offset        [host] step counter folded into the Philox counter
 * B, K, V       1 <= B <= SV_MAX_BATCH, 0 <= K <= SV_MAX_DRAFT,
 *               1 <= V <= SV_MAX_VOCAB
 * out_tokens    [B, K+1] int32: accepted drafts, then the drawn token,
 *               then -1
 * out_accept_len [B] int32: tokens emitted, a + 1 in [1, K+1]
 * out_p_draft   [B, K] float or NULL: p_i(x_i) for every i < K
 * out_q_draft   [B, K] float or NULL: q_i(x_i) for every i < K
 * Device-side values: a request whose temperature is not a finite positive
 * number is refused (accept_len 0, tokens -1, p/q 0); a draft token outside
 * [0, V) has p = q = 0 and is rejected; logits must not be NaN or +inf and
 * a row must not be entirely -inf (results are then unspecified, never an
 * out-of-bounds access).
 */
int spec_verify_sample(const sv_logits* target, const sv_logits* draft,
                       const int32_t* draft_tokens, const float* temperature,
                       const uint64_t* seeds, uint64_t offset,
                       int32_t B, int32_t K, int32_t V,
                       int32_t* out_tokens, int32_t* out_accept_len,
                       float* out_p_draft, float* out_q_draft,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy (argmax-match) verification: g_i = argmax_v target[b, i, v]
 * (lowest index on ties); the longest prefix with draft_tokens[b, i] == g_i
 * is accepted (a tokens) and g_a is emitted after it. This reproduces plain
 * greedy decoding ("推测解码与 MTP" §11; MTP drafts, §6.2).
 *
 * target [B, K+1, V]; draft_tokens [B, K] (may be NULL when K == 0);
 * out_tokens [B, K+1] (-1 padded); out_accept_len [B] in [1, K+1];
 * out_argmax [B, K+1] or NULL (g_i of every row). Limits as for sampling.
 * A draft token outside [0, V) never matches.
 */
int spec_verify_greedy(const sv_logits* target, const int32_t* draft_tokens,
                       int32_t B, int32_t K, int32_t V,
                       int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k / top-p filtered stochastic verification. The pages run speculative
 * decoding with the sampler's parameters (temperature 0.8, top_p 0.95, in
 * "Speculative Decoding Guide", vLLM-Ascend), so p and q are the filtered
 * distributions the sampler draws from: for each target row and, with draft
 * logits, each draft row, after the temperature:
 *   top-k: keep the logits at least the k-th largest (ties at the cut kept);
 *          top_k[b] <= 0 or >= V keeps all;
 *   top-p: of those, keep the logits at least t, where t is the largest
 *          logit value whose upper set {l >= t} holds at least top_p[b] of
 *          their mass (ties kept); top_p[b] >= 1 (or NaN) keeps all;
 * then renormalise, and run the rule of spec_verify_sample on the filtered
 * rows. One-hot drafts stay one-hot. top_k and top_p are device arrays [B]
 * (int32, fp32); either may be NULL (that filter off for every request).
 * Precision of the cut: bf16 rows count every distinct value, so the cut is
 * exact at any depth (masses are counts times fp64 weights); fp32 rows find
 * it exactly among logits whose weight is within 2^-64 of the row's largest,
 * and a cut below that keeps the whole row. out_p_draft / out_q_draft hold
 * the filtered p_i(x_i) / q_i(x_i). fp32 rows only: when both are NULL,
 * drafts are one-hot and top-k is off for a request, rows past its first
 * certain rejection (u * top_p >= p_j(x_j), which rejects whatever the cut)
 * are not cut: the tokens and accept lengths are the same, the call is
 * faster. Other arguments, limits and errors as spec_verify_sample; the
 * workspace is sized as for it.
 */
int spec_verify_sample_filtered(const sv_logits* target, const sv_logits* draft,
                                const int32_t* draft_tokens, const float* temperature,
                                const int32_t* top_k, const float* top_p,
                                const uint64_t* seeds, uint64_t offset,
                                int32_t B, int32_t K, int32_t V,
                                int32_t* out_tokens, int32_t* out_accept_len,
                                float* out_p_draft, float* out_q_draft,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_sample without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The call's workspace is a static
 * device array of 16 MiB (SV_NOALLOC_SCRATCH_BYTES) inside the library; each
 * device the library runs on holds its own copy until the process ends.
 * The call allocates nothing; its first call on a device (with that device
 * current, `stream` on it) looks the array's address up once and zero-fills
 * it on `stream`. Calls leave its counter and tagged words zero again, so
 * every call starts clean; the array keeps the rest of the last call's
 * contents. All such calls on one device share the one array: calls that
 * may overlap on a device (different streams, different threads) race, and
 * must be serialised by the caller.
 * Arguments, results and errors are those of spec_verify_sample; a call
 * whose workspace (spec_verify_workspace_size) would exceed the scratch
 * returns SV_ERR_SCRATCH before anything is launched (B=256, K=5, V=128256
 * one-hot needs 7.1 MiB).
 */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_sample_noalloc(const sv_logits* target, const sv_logits* draft,
                               const int32_t* draft_tokens, const float* temperature,
                               const uint64_t* seeds, uint64_t offset,
                               int32_t B, int32_t K, int32_t V,
                               int32_t* out_tokens, int32_t* out_accept_len,
                               float* out_p_draft, float* out_q_draft, void* stream);

/*
 * Early-exit ("lazy") stochastic verification. The rule stops at the first
 * rejection ("推测解码与 MTP" §2.1), so the rows after it are not needed.
 * This call reads two position-major rounds: position 0, then positions
 * 1..K. A round reads the window's target rows (and draft rows) only of the
 * requests still open after the previous round, and decides its positions
 * in order. A request that stops at position 0 has read only its row 0
 * (and draft row 0); one that goes on reads all its rows. It pays off when
 * most drafts are rejected at the first position. Tokens, accept
 * lengths and the uniforms used are those of spec_verify_sample;
 * out_p_draft / out_q_draft hold p_i(x_i) / q_i(x_i) up to the stop
 * position and 0 after it. Arguments, limits and errors as
 * spec_verify_sample; the workspace is sized as for it.
 */
int spec_verify_sample_lazy(const sv_logits* target, const sv_logits* draft,
                            const int32_t* draft_tokens, const float* temperature,
                            const uint64_t* seeds, uint64_t offset,
                            int32_t B, int32_t K, int32_t V,
                            int32_t* out_tokens, int32_t* out_accept_len,
                            float* out_p_draft, float* out_q_draft,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grammar-constrained verification (LMDeploy "Speculative Decoding",
 * structured output: the grammar mask is applied to the target's logits at
 * every verified position before rejection sampling; drafts were proposed
 * under the same masks).
 *
 * bitmask       [B, K+1, ceil(V/32)] uint32, row-major: token v is allowed at
 *               position i of request b when bit v % 32 of word
 *               bitmask[b, i, v / 32] is 1. Disallowed logits of target row i
 *               and, with draft logits, draft row i count as -inf; the rule
 *               is then exactly spec_verify_sample / spec_verify_greedy on the
 *               masked logits. A draft token that is disallowed has p = 0 and
 *               is rejected; drawn tokens are always allowed.
 * Every other argument as in spec_verify_sample / spec_verify_greedy; a
 * position with no allowed token is a caller error (results unspecified,
 * never an out-of-bounds access). SV_ERR_NULL for a NULL bitmask.
 */
int spec_verify_sample_masked(const sv_logits* target, const sv_logits* draft,
                              const int32_t* draft_tokens, const uint32_t* bitmask,
                              const float* temperature, const uint64_t* seeds, uint64_t offset,
                              int32_t B, int32_t K, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_p_draft, float* out_q_draft,
                              void* workspace, size_t workspace_bytes, void* stream);

int spec_verify_greedy_masked(const sv_logits* target, const int32_t* draft_tokens,
                              const uint32_t* bitmask, int32_t B, int32_t K, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged batches: every request has its own draft count K_b (a verifier
 * takes variable-length queries from one forward and maps each output row
 * back to its request: FastDeploy "投机解码", framework design, virtual
 * padding; adaptive per-request draft counts: vLLM-Ascend "Speculative
 * Decoding Guide", suffix decoding; "推测解码与 MTP" §10.2).
 *
 * Rows are packed. With cu = cu_draft (device, [B + 1] int32 prefix sums,
 * K_b = cu[b + 1] - cu[b]):
 *   target rows of request b: packed rows cu[b] + b ... cu[b] + b + K_b of
 *     `target` ([total_k + B, V]; rows stride_k apart, stride_b unused);
 *   draft rows (explicit q): packed rows cu[b] ... cu[b] + K_b - 1 of
 *     `draft` ([total_k, V]), or NULL for one-hot q;
 *   draft tokens: draft_tokens[cu[b] ... cu[b] + K_b - 1] ([total_k]);
 *   out_p_draft / out_q_draft: [total_k] at the same positions;
 *   out_tokens: [B, K_max + 1], columns past K_b are -1;
 *   out_argmax (greedy): [total_k + B] at the target rows' positions.
 * The rule per request is the dense one with K = K_b, with the uniforms of
 * (seeds[b], b, position): a ragged call equals the dense call on each
 * request's own rows. total_k [host] is the number of packed drafts and
 * K_max [host] (0..SV_MAX_DRAFT) bounds every K_b; the workspace is sized
 * as for the dense call with K = K_max.
 * Device-side checks: a request with cu[b] < 0, cu[b + 1] < cu[b],
 * cu[b + 1] > total_k or K_b > K_max is refused (accept_len 0, tokens -1)
 * and none of its rows is read; every row read lies in the ranges above.
 * Other device values behave as in the dense calls. Host errors: as the
 * dense calls, plus SV_ERR_NULL for a NULL cu_draft (or NULL draft_tokens
 * with total_k > 0) and SV_ERR_SHAPE for total_k < 0.
 */
int spec_verify_sample_ragged(const sv_logits* target, const sv_logits* draft,
                              const int32_t* cu_draft, int32_t total_k,
                              const int32_t* draft_tokens, const float* temperature,
                              const uint64_t* seeds, uint64_t offset,
                              int32_t B, int32_t K_max, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len,
                              float* out_p_draft, float* out_q_draft,
                              void* workspace, size_t workspace_bytes, void* stream);

int spec_verify_greedy_ragged(const sv_logits* target, const int32_t* cu_draft, int32_t total_k,
                              const int32_t* draft_tokens, int32_t B, int32_t K_max, int32_t V,
                              int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_argmax,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy verification of a static draft tree (Medusa, "推测解码与 MTP"
 * §3.3: every node attends only to its ancestors; the longest accepted
 * root path wins).
 *
 * target       [B, N, V]: row n holds the logits the target produced at
 *              node n (its prediction for the token after node n)
 * node_tokens  [B, N] int32: the draft token of each node (column 0, the
 *              root, is ignored)
 * parents      [host] [N] int32: parents[0] == -1, 0 <= parents[n] < n
 * N, B, V      2 <= N <= SV_MAX_TREE_NODES; B, V as above
 * Node n != 0 is accepted when its parent is accepted and
 * node_tokens[b, n] == argmax(row parents[n]) (lowest index on ties); the
 * deepest accepted node wins (lowest index on ties).
 * out_tokens     [B, N] int32: the winning path's node tokens (root
 *                excluded), then the winner's argmax, then -1
 * out_accept_len [B] int32: depth(best) + 1
 * out_best_node  [B] int32 or NULL
 * SV_ERR_TREE when `parents` is malformed.
 */
int spec_verify_tree(const sv_logits* target, const int32_t* node_tokens,
                     const int32_t* parents, int32_t N, int32_t B, int32_t V,
                     int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_best_node,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy verification of dynamic draft trees: a tree per request, as the
 * drafter builds it for each context (EAGLE-2, "推测解码与 MTP" §4.3: the
 * best tree differs by position and context, so each step keeps only the
 * most promising nodes). The rule per request is spec_verify_tree's.
 *
 * parents      [B, N] int32, device, row-major: request b's tree is row b,
 *              with parents[b, 0] == -1 and 0 <= parents[b, n] < n
 * Every other argument, output and host error as spec_verify_tree (the
 * workspace of SV_OP_TREE with the same B, N, V). The rows are checked on
 * the device: a request whose row is not such a tree is refused
 * (out_accept_len 0, out_tokens -1, out_best_node -1) and the others are
 * verified as usual.
 */
int spec_verify_tree_dynamic(const sv_logits* target, const int32_t* node_tokens,
                             const int32_t* parents, int32_t N, int32_t B, int32_t V,
                             int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_best_node,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* spec_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
