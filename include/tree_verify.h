/*
 * tree_verify.h — C ABI of the MI355X (gfx950) tree-verification library.
 *
 * One speculative-decoding verify step over a flattened draft tree of N
 * nodes, described by tokens[N], parent[N] (-1 = child of the last accepted
 * token) and optionally depth[N], flattened spine-first per depth
 * (serve-integration spec "tree_dev/SERVE_INTEGRATION_SPEC.md", section
 * "Layout contract").
 *
 * Conventions shared by every entry point
 *  - Array arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Arrays are dense, row-major, in
 *    the layout stated per argument.
 *  - State: the library keeps only per-device caches, filled on its first
 *    call on a device and written with atomics (safe across host threads):
 *    the device's compute-unit and XCD counts (which size some grids), flags
 *    recording that the dynamic-LDS limit of a kernel was raised with
 *    hipFuncSetAttribute on that device, and the device address of the static
 *    scratch of tree_walk_accept_noalloc.  No call depends on an earlier
 *    call's data.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call enqueues its kernels on that stream and returns at once.
 *  - Argument errors (null pointers, shapes, unsupported sizes or dtypes,
 *    a workspace that is too small) are detected on the host before anything
 *    is launched and returned as a tv_status; nothing is enqueued then.
 *    Data-dependent errors (a malformed tree) are reported per sequence in a
 *    device status array by tree_mask_build.  TV_ERR_LAUNCH reports a failed
 *    kernel launch.
 *  - Floating-point inputs are either all fp32 (TV_F32) or all bf16
 *    (TV_BF16) per call, except where an argument says fp32; accumulation is
 *    fp32.  Outputs are fp32 or, for bf16 inputs, bf16 (`out_dtype`); a bf16
 *    output is the fp32 result rounded to nearest even.
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TV_OK = 0,
  TV_ERR_NULL = 1,        /* a required pointer is NULL                      */
  TV_ERR_SHAPE = 2,       /* inconsistent or non-positive sizes              */
  TV_ERR_UNSUPPORTED = 3, /* sizes or dtype outside the supported set        */
  TV_ERR_WORKSPACE = 4,   /* workspace pointer NULL or smaller than required */
  TV_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch        */
  TV_ERR_SCRATCH = 6      /* input larger than the library's static scratch  */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Per-sequence device status written by tree_mask_build. */
enum {
  TV_TREE_OK = 0,
  TV_TREE_BAD_PARENT = 1, /* some parent[i] outside [-1, i)                   */
  TV_TREE_BAD_DEPTH = 2,  /* depth_in given and different from the derived one */
  TV_TREE_BAD_CTX = 3     /* ctx_len < 1                                      */
};

typedef void* tv_stream;

#define TV_MAX_NODES 128     /* draft nodes per tree (mask, attention, walk, KV commit) */
#define TV_GDN_MAX_NODES 128 /* draft nodes per tree for the Gated DeltaNet calls       */
#define TV_BLOCK_SIZE 16     /* tokens per KV-cache page                                */
#define TV_TREE_MAX_TOPK 16  /* candidates per depth for tree construction             */
#define TV_TREE_MAX_DEPTH 16 /* depths of a constructed tree                           */
/* 64-bit words of one node's ancestor set: node j is bit j % 64 of word j / 64 */
#define TV_ANC_WORDS(N) (((N) + 63) / 64)

/* ------------------------------------------------------------------------
 * tree_mask_build — ancestor-or-self mask, depths and position ids.
 *
 * Serve-integration spec, section "2. Verify: tree attention mask": a node
 * sees, among draft nodes, only its ancestors and itself, and its position id
 * is ctx_len - 1 + depth.  Depth is 1 for a node whose parent is -1 (DDTree
 * validation post "From Linear to Tree-Walk", section "The Successful Test",
 * printed depths and parents).
 *
 *   parent       int32 [B, N]   parent node index, -1 = under the last accepted token
 *   depth_in     int32 [B, N]   optional (NULL): proposer depths, checked against
 *                               the derived ones
 *   ctx_len      int32 [B]      committed tokens per sequence (the last accepted
 *                               token included, at position ctx_len - 1)
 *   anc_mask     uint64 [B, N, TV_ANC_WORDS(N)]  out: bit j % 64 of word j / 64
 *                               set iff node j is node t or an ancestor of t
 *   depth_out    int32 [B, N]   out: derived depth (1 = child of the root)
 *   position_ids int32 [B, N]   out: ctx_len[b] - 1 + depth
 *   dense_bias   float [B, N, N] optional out (NULL = skip): 0 where anc bit set,
 *                               -inf elsewhere (the additive node-block bias)
 *   status       int32 [B]      out: TV_TREE_* of each sequence; checks apply in
 *                               the order parent, depth, ctx and the first failure
 *                               is reported.  With TV_TREE_BAD_PARENT the outputs
 *                               of that sequence are those of a star (each node
 *                               sees only itself, depth 1); otherwise the derived
 *                               values are written even when the status is nonzero.
 * Supported: 1 <= N <= TV_MAX_NODES, B >= 1.
 * ------------------------------------------------------------------------ */
tv_status tree_mask_build(const int32_t* parent, const int32_t* depth_in,
                          const int32_t* ctx_len, int32_t B, int32_t N,
                          uint64_t* anc_mask, int32_t* depth_out,
                          int32_t* position_ids, float* dense_bias,
                          int32_t* status, tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_verify_attn — tree-masked attention of the N draft nodes over the
 * paged context plus their ancestors.
 *
 * Serve-integration spec, section "2. Verify: tree attention mask": every
 * node attends to all committed context keys and, among the nodes, only to
 * its ancestors and itself; the mask composes with the layer's sliding
 * window.  A key at position k is visible to a query at position p iff
 * 0 <= p - k < window (window <= 0: no window); node keys use their own
 * position ids.  Query head h reads kv head h / (Hq / Hkv).  Scores are
 * scale * <q, k> (q and k already rotated; no soft cap).
 *
 *   q            [B, N, Hq, D]           queries of the draft nodes
 *   k_node       [B, N, Hkv, D]          keys of the draft nodes
 *   v_node       [B, N, Hkv, D]          values of the draft nodes
 *   k_cache      [num_blocks, Hkv, 16, D] paged context keys (one page holds 16
 *                                        consecutive positions of one sequence)
 *   v_cache      [num_blocks, Hkv, 16, D] paged context values
 *   block_table  int32 [B, max_blocks_per_seq]  page of positions 16j..16j+15
 *   ctx_len      int32 [B]               context length (<= max_ctx_len)
 *   max_ctx_len  host bound on ctx_len, <= 16 * max_blocks_per_seq; sizes the grid
 *   anc_mask     uint64 [B, N, TV_ANC_WORDS(N)]  from tree_mask_build
 *   position_ids int32 [B, N]            from tree_mask_build
 *   out          [B, N, Hq, D]           attention output, in out_dtype
 *   workspace    device scratch of tree_verify_attn_workspace_size(...) bytes
 *                (contents on entry do not matter; it holds split partials)
 * Page indices outside [0, num_blocks) and ctx_len outside [0, max_ctx_len]
 * are clamped into range (the output is then unspecified, but no access
 * leaves the buffers).
 * Supported: 1 <= N <= TV_MAX_NODES, D in {64, 128, 256}, block_size == 16,
 * Hq % Hkv == 0, dtype TV_F32 or TV_BF16 (out_dtype TV_F32, or TV_BF16 with
 * bf16 inputs), Hq / Hkv * N <= 4096, 0 < scale < infinity.
 * ------------------------------------------------------------------------ */
size_t tree_verify_attn_workspace_size(int32_t B, int32_t N, int32_t Hq,
                                       int32_t Hkv, int32_t D,
                                       int32_t max_ctx_len, int32_t window);

tv_status tree_verify_attn(const void* q, const void* k_node, const void* v_node,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t num_blocks, const int32_t* ctx_len,
                           int32_t max_ctx_len, const uint64_t* anc_mask,
                           const int32_t* position_ids, int32_t B, int32_t N,
                           int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                           int32_t window, float scale, tv_dtype dtype,
                           tv_dtype out_dtype, void* out, void* workspace,
                           size_t workspace_bytes, tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_gdn_verify — Gated DeltaNet outputs of every draft node, with no
 * state written.
 *
 * DFlash-TfM summary (gist.science, "Trees from Marginals"), section
 * "3. Rollback-vrije Boom-verificatie voor GDN": along each node's root path
 * the state follows S_t = alpha_t (I - beta_t k_t k_t^T) S_parent
 * + beta_t k_t v_t^T from the committed state S0; the output is
 * o_t = S_t^T q_t.  The library evaluates it as the section's masked
 * triangular solve over the ancestor interaction matrices and never writes a
 * state (the commit happens after the walk, outside this call).
 *
 *   q, k      [B, N, H, Dk]   dtype
 *   v         [B, N, H, Dv]   dtype
 *   alpha     float [B, N, H] gates
 *   beta      float [B, N, H] write strengths
 *   S0        float [B, H, Dk, Dv] committed state (read only)
 *   anc_mask  uint64 [B, N, TV_ANC_WORDS(N)]  from tree_mask_build
 *   out       [B, N, H, Dv]   out_dtype (TV_F32, or TV_BF16 with bf16 inputs)
 * Gates may be any finite values, 0 included (a gate exp(g) that underflowed):
 * a zero gate cuts the path's decay products to exactly 0.
 * q, k, v, S0 and out must be 16-byte aligned.
 * Supported: 1 <= N <= TV_GDN_MAX_NODES, Dk == Dv == 128.
 * ------------------------------------------------------------------------ */
tv_status tree_gdn_verify(const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, const float* S0,
                          const uint64_t* anc_mask, int32_t B, int32_t N, int32_t H,
                          int32_t Dk, int32_t Dv, tv_dtype dtype, tv_dtype out_dtype,
                          void* out, tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_walk_accept — greedy tree walk with the bonus token.
 *
 * Serve-integration spec, sections "What's proven" and "3. Rejection
 * sampler: tree walk": from the root (the last accepted token) follow the
 * child whose token equals the target argmax at the current node; when none
 * matches, emit that argmax as the bonus token.  Row 0 of the logits belongs
 * to the root, row 1 + i to node i.  The argmax takes the lowest index among
 * equal maxima; among several matching children the lowest index wins.
 * Logits must be finite (otherwise the result is unspecified).
 *
 *   tokens          int32 [B, N]      draft tokens (values outside [0, V) never match)
 *   parent          int32 [B, N]      as for tree_mask_build; a node whose parent
 *                                     is outside [-1, i) never matches
 *   logits          [B, N + 1, V]     dtype
 *   accepted_tokens int32 [B, N + 1]  out: a accepted tokens then the bonus, then -1
 *   accepted_nodes  int32 [B, N]      out: the a accepted node indices, then -1
 *   num_accepted    int32 [B]         out: a
 *   workspace       tree_walk_accept_workspace_size(B, N) bytes of device scratch
 * Supported: 1 <= N <= TV_MAX_NODES, V >= 1.
 * ------------------------------------------------------------------------ */
size_t tree_walk_accept_workspace_size(int32_t B, int32_t N);

tv_status tree_walk_accept(const int32_t* tokens, const int32_t* parent,
                           const void* logits, int32_t B, int32_t N, int32_t V,
                           tv_dtype dtype, int32_t* accepted_tokens,
                           int32_t* accepted_nodes, int32_t* num_accepted,
                           void* workspace, size_t workspace_bytes,
                           tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_walk_accept_noalloc — tree_walk_accept for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.
 *
 * Same arguments (without the workspace) and the same results as
 * tree_walk_accept.  The per-row argmax goes to a static device array of
 * TV_WALK_NOALLOC_MAX_ROWS int32 (1 MiB) inside the library; each GPU the
 * library runs on holds its own copy until the process ends.  The call
 * allocates nothing: its first call on a device only looks up that array's
 * device address (hipGetSymbolAddress) and keeps it.  Every row is written
 * before it is read, so the array's contents from earlier calls do not
 * matter.  Calls that overlap on one GPU (other streams, other host threads)
 * share the array and race: serialise them.
 * B * (N + 1) > TV_WALK_NOALLOC_MAX_ROWS returns TV_ERR_SCRATCH before
 * anything is launched.
 * ------------------------------------------------------------------------ */
#define TV_WALK_NOALLOC_MAX_ROWS 262144

tv_status tree_walk_accept_noalloc(const int32_t* tokens, const int32_t* parent,
                                   const void* logits, int32_t B, int32_t N, int32_t V,
                                   tv_dtype dtype, int32_t* accepted_tokens,
                                   int32_t* accepted_nodes, int32_t* num_accepted,
                                   tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_gdn_commit — the Gated DeltaNet state after the walk.
 *
 * DFlash-TfM summary (gist.science, "Trees from Marginals"), section
 * "3. Rollback-vrije Boom-verificatie voor GDN": the verify pass writes no
 * state; once the accepted branch is known, the committed state advances
 * along it by S <- alpha_t (I - beta_t k_t k_t^T) S + beta_t k_t v_t^T for
 * the accepted nodes t in order (the first a child of the last accepted
 * token).  With no accepted node the state stays S0.
 *
 *   k          [B, N, H, Dk]   dtype (the verify pass's keys)
 *   v          [B, N, H, Dv]   dtype
 *   alpha      float [B, N, H] gates
 *   beta       float [B, N, H] write strengths
 *   S0         float [B, H, Dk, Dv] committed state before the step
 *   accepted_nodes int32 [B, N]  from tree_walk_accept (first num_accepted
 *                                entries used; indices are clamped into [0, N))
 *   num_accepted   int32 [B]     from tree_walk_accept (clamped into [0, N])
 *   S_out      float [B, H, Dk, Dv] out: the new committed state; may be S0
 *              itself (each (sequence, head) block is read before it is written)
 * k, v, S0 and S_out must be 16-byte aligned.
 * Supported: 1 <= N <= TV_GDN_MAX_NODES, Dk == Dv == 128, dtype TV_F32 or TV_BF16.
 * ------------------------------------------------------------------------ */
tv_status tree_gdn_commit(const void* k, const void* v, const float* alpha,
                          const float* beta, const float* S0,
                          const int32_t* accepted_nodes, const int32_t* num_accepted,
                          int32_t B, int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                          tv_dtype dtype, float* S_out, tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_kv_commit — the accepted path's keys and values into the paged cache.
 *
 * Serve-integration spec, layout contract and "3. Rejection sampler: tree
 * walk": accepted node s (depth s + 1) has position id ctx_len - 1 + depth =
 * ctx_len + s.  Its key and value rows of every kv head, as the verify pass
 * computed them, are copied bit for bit into slot (ctx_len + s) % 16 of page
 * block_table[b][(ctx_len + s) / 16].  The caller allocates the pages; no
 * other cache entry changes.
 *
 *   k_node, v_node [B, N, Hkv, D]   dtype, as given to tree_verify_attn
 *   accepted_nodes int32 [B, N], num_accepted int32 [B]  from tree_walk_accept
 *   ctx_len        int32 [B]        context length before the step
 *   block_table    int32 [B, max_blocks_per_seq]
 *   k_cache, v_cache [num_blocks, Hkv, 16, D]  dtype, updated in place
 * Entries past num_accepted, node indices outside [0, N), negative positions
 * and positions whose page index lies outside the table or the pool are not
 * written.  All four K/V pointers must be 16-byte aligned.
 * Supported: 1 <= N <= TV_MAX_NODES, D in {64, 128, 256}, block_size == 16,
 * dtype TV_F32 or TV_BF16.
 * ------------------------------------------------------------------------ */
tv_status tree_kv_commit(const void* k_node, const void* v_node,
                         const int32_t* accepted_nodes, const int32_t* num_accepted,
                         const int32_t* ctx_len, const int32_t* block_table,
                         int32_t max_blocks_per_seq, int32_t num_blocks, int32_t B,
                         int32_t N, int32_t Hkv, int32_t D, int32_t block_size,
                         tv_dtype dtype, void* k_cache, void* v_cache, tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_draft_topk — the candidates of each depth of a factorised draft.
 *
 * DDTree validation post ("From Linear to Tree-Walk"), section "The Failed
 * First Attempt": the tree starts from the top-k tokens of the first
 * position, and every depth offers its top-k tokens with their draft
 * log-probabilities.  For each (sequence b, depth d) row of draft logits the
 * call returns the K largest logits' token ids (ties to the lower id) in
 * decreasing order and their log-softmax values over the whole row.
 *
 *   logits        [B, L, V]   dtype, row (b, d) = draft logits of depth d + 1
 *   cand_tokens   int32 [B, L, K]  out
 *   cand_logprob  float [B, L, K]  out: logit - log(sum over the row of exp(logit))
 * Logits must be finite (otherwise the result is unspecified).
 * Supported: B >= 1, 1 <= L <= TV_TREE_MAX_DEPTH, 1 <= K <= TV_TREE_MAX_TOPK,
 * K <= V, dtype TV_F32 or TV_BF16.
 * ------------------------------------------------------------------------ */
tv_status tree_draft_topk(const void* logits, int32_t B, int32_t L, int32_t V, int32_t K,
                          tv_dtype dtype, int32_t* cand_tokens, float* cand_logprob,
                          tv_stream stream);

/* ------------------------------------------------------------------------
 * tree_build — best-first growth of the draft tree from per-depth candidates.
 *
 * DDTree validation post, section "The Failed First Attempt": a priority
 * queue on cumulative log-probability starts with the depth-1 candidates as
 * roots; each popped node joins the tree and its sibling and child are
 * queued, until the budget N is spent or the maximum depth L stops growth.
 * DFlash-TfM summary, section "2. Boomconstructie": each round takes the w
 * best candidates at once and expands them together (ceil(N / w) rounds).
 * Precisely: the queue starts with the K depth-1 candidates in rank order; a
 * node's value is its parent's value plus its candidate's log-probability,
 * one float32 addition; the queue orders by value, higher first, equal
 * values in push order; a round pops min(w, N - nodes so far, queued)
 * candidates in queue order, then pushes, for each popped node in pop order,
 * its next sibling (same parent, next rank; depth >= 2 only, depth-1
 * siblings are queued from the start) and its first child (rank 0 of the
 * next depth, below depth L).  Output order: pop order stable-sorted by
 * depth (the best node of each depth first), parents renumbered; parent -1 is
 * a child of the last accepted token, depth 1 its depth (the layout contract
 * of tree_mask_build).
 *
 *   cand_tokens   int32 [B, L, K], cand_logprob float [B, L, K]  (as from
 *                 tree_draft_topk; log-probabilities in decreasing order per depth)
 *   tokens        int32 [B, N]  out: node tokens (-1 past the tree)
 *   parent        int32 [B, N]  out: parent node (-1 for depth 1 and past the tree)
 *   depth         int32 [B, N]  out: 1-based depth (0 past the tree)
 *   score         float [B, N]  optional out (NULL = skip): cumulative log-probability
 *   num_nodes     int32 [B]     out: nodes built (N unless the K-ary tree of depth L is smaller)
 * Supported: B >= 1, 1 <= L <= TV_TREE_MAX_DEPTH, 1 <= K <= TV_TREE_MAX_TOPK,
 * 1 <= N <= TV_MAX_NODES, w >= 1.
 * ------------------------------------------------------------------------ */
tv_status tree_build(const int32_t* cand_tokens, const float* cand_logprob, int32_t B,
                     int32_t L, int32_t K, int32_t N, int32_t w, int32_t* tokens,
                     int32_t* parent, int32_t* depth, float* score, int32_t* num_nodes,
                     tv_stream stream);

/* Static description of a status code. */
const char* tv_status_string(tv_status s);

#ifdef __cplusplus
}
#endif

#endif /* TREE_VERIFY_H */
