// C ABI of the tree-verification library: argument validation on the host,
// then the kernel launches.  Nothing here allocates, frees or synchronises.
#include "tv_internal.h"

namespace {

hipStream_t as_stream(tv_stream s) { return reinterpret_cast<hipStream_t>(s); }

tv_status launched(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_LAUNCH; }

bool dtype_ok(tv_dtype d) { return d == TV_F32 || d == TV_BF16; }

// outputs are fp32, or bf16 when the inputs are bf16
bool out_dtype_ok(tv_dtype in, tv_dtype out) {
  return out == TV_F32 || (out == TV_BF16 && in == TV_BF16);
}

constexpr int kMaxRowsPerKvHead = 4096;  // (Hq / Hkv) * N

}  // namespace

extern "C" {

const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_SHAPE: return "inconsistent or non-positive sizes";
    case TV_ERR_UNSUPPORTED: return "sizes or dtype outside the supported set";
    case TV_ERR_WORKSPACE: return "workspace missing or too small";
    case TV_ERR_LAUNCH: return "kernel launch failed";
    case TV_ERR_SCRATCH: return "input larger than the library's static scratch";
  }
  return "unknown status";
}

tv_status tree_mask_build(const int32_t* parent, const int32_t* depth_in, const int32_t* ctx_len,
                          int32_t B, int32_t N, uint64_t* anc_mask, int32_t* depth_out,
                          int32_t* position_ids, float* dense_bias, int32_t* status,
                          tv_stream stream) {
  if (!parent || !ctx_len || !anc_mask || !depth_out || !position_ids || !status)
    return TV_ERR_NULL;
  if (B < 1 || N < 1) return TV_ERR_SHAPE;
  if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
  return launched(tv::launch_mask(parent, depth_in, ctx_len, B, N, anc_mask, depth_out,
                                  position_ids, dense_bias, status, as_stream(stream)));
}

size_t tree_verify_attn_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t max_ctx_len, int32_t window) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_ctx_len < 0) return 0;
  return tv::attn_plan(B, N, Hq, Hkv, D, max_ctx_len, window).ws_bytes;
}

tv_status tree_verify_attn(const void* q, const void* k_node, const void* v_node,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           int32_t max_blocks_per_seq, int32_t num_blocks, const int32_t* ctx_len,
                           int32_t max_ctx_len, const uint64_t* anc_mask,
                           const int32_t* position_ids, int32_t B, int32_t N, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t block_size, int32_t window, float scale,
                           tv_dtype dtype, tv_dtype out_dtype, void* out, void* workspace,
                           size_t workspace_bytes, tv_stream stream) {
  if (!q || !k_node || !v_node || !ctx_len || !anc_mask || !position_ids || !out)
    return TV_ERR_NULL;
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || max_ctx_len < 0 || max_blocks_per_seq < 0 ||
      num_blocks < 0)
    return TV_ERR_SHAPE;
  if (Hq % Hkv != 0) return TV_ERR_SHAPE;
  if (static_cast<long long>(max_ctx_len) > 16LL * max_blocks_per_seq) return TV_ERR_SHAPE;
  if (max_ctx_len > 0 && (!k_cache || !v_cache || !block_table)) return TV_ERR_NULL;
  if (max_ctx_len > 0 && num_blocks < 1) return TV_ERR_SHAPE;
  if (!dtype_ok(dtype) || !out_dtype_ok(dtype, out_dtype)) return TV_ERR_UNSUPPORTED;
  if (N > TV_MAX_NODES || block_size != TV_BLOCK_SIZE) return TV_ERR_UNSUPPORTED;
  if (D != 64 && D != 128 && D != 256) return TV_ERR_UNSUPPORTED;
  // a softmax scale is positive and finite (the kernels take row maxima on the
  // unscaled scores)
  if (!(scale > 0.0f) || !(scale < INFINITY)) return TV_ERR_UNSUPPORTED;
  if (static_cast<long long>(Hq / Hkv) * N > kMaxRowsPerKvHead) return TV_ERR_UNSUPPORTED;
  const tv::AttnPlan plan = tv::attn_plan(B, N, Hq, Hkv, D, max_ctx_len, window);
  if (plan.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.ws_bytes))
    return TV_ERR_WORKSPACE;
  return launched(tv::launch_attn(plan, q, k_node, v_node, k_cache, v_cache, block_table,
                                  max_blocks_per_seq, num_blocks, ctx_len, max_ctx_len, anc_mask,
                                  position_ids, B, N, Hq, Hkv, D, window, scale, dtype, out_dtype,
                                  out, workspace, as_stream(stream)));
}

tv_status tree_gdn_verify(const void* q, const void* k, const void* v, const float* alpha,
                          const float* beta, const float* S0, const uint64_t* anc_mask, int32_t B,
                          int32_t N, int32_t H, int32_t Dk, int32_t Dv, tv_dtype dtype,
                          tv_dtype out_dtype, void* out, tv_stream stream) {
  if (!q || !k || !v || !alpha || !beta || !S0 || !anc_mask || !out) return TV_ERR_NULL;
  if (B < 1 || N < 1 || H < 1 || Dk < 1 || Dv < 1) return TV_ERR_SHAPE;
  if (!dtype_ok(dtype) || !out_dtype_ok(dtype, out_dtype)) return TV_ERR_UNSUPPORTED;
  if (N > TV_GDN_MAX_NODES || Dk != 128 || Dv != 128) return TV_ERR_UNSUPPORTED;
  // rows of q, k, v, the state and the output move in 16-byte pieces
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(S0) |
                          reinterpret_cast<uintptr_t>(out);
  if (align & 15u) return TV_ERR_UNSUPPORTED;
  return launched(tv::launch_gdn(q, k, v, alpha, beta, S0, anc_mask, B, N, H, Dk, Dv, dtype,
                                 out_dtype, out, as_stream(stream)));
}

tv_status tree_gdn_commit(const void* k, const void* v, const float* alpha, const float* beta,
                          const float* S0, const int32_t* accepted_nodes,
                          const int32_t* num_accepted, int32_t B, int32_t N, int32_t H, int32_t Dk,
                          int32_t Dv, tv_dtype dtype, float* S_out, tv_stream stream) {
  if (!k || !v || !alpha || !beta || !S0 || !accepted_nodes || !num_accepted || !S_out)
    return TV_ERR_NULL;
  if (B < 1 || N < 1 || H < 1 || Dk < 1 || Dv < 1) return TV_ERR_SHAPE;
  if (!dtype_ok(dtype)) return TV_ERR_UNSUPPORTED;
  if (N > TV_GDN_MAX_NODES || Dk != 128 || Dv != 128) return TV_ERR_UNSUPPORTED;
  // the state and the key/value rows move in 16-byte pieces
  const uintptr_t align = reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                          reinterpret_cast<uintptr_t>(S0) | reinterpret_cast<uintptr_t>(S_out);
  if (align & 15u) return TV_ERR_UNSUPPORTED;
  return launched(tv::launch_gdn_commit(k, v, alpha, beta, S0, accepted_nodes, num_accepted, B, N,
                                        H, dtype, S_out, as_stream(stream)));
}

tv_status tree_kv_commit(const void* k_node, const void* v_node, const int32_t* accepted_nodes,
                         const int32_t* num_accepted, const int32_t* ctx_len,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         int32_t num_blocks, int32_t B, int32_t N, int32_t Hkv, int32_t D,
                         int32_t block_size, tv_dtype dtype, void* k_cache, void* v_cache,
                         tv_stream stream) {
  if (!k_node || !v_node || !accepted_nodes || !num_accepted || !ctx_len || !block_table ||
      !k_cache || !v_cache)
    return TV_ERR_NULL;
  if (B < 1 || N < 1 || Hkv < 1 || D < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
    return TV_ERR_SHAPE;
  if (!dtype_ok(dtype) || block_size != TV_BLOCK_SIZE) return TV_ERR_UNSUPPORTED;
  if (N > TV_MAX_NODES || (D != 64 && D != 128 && D != 256)) return TV_ERR_UNSUPPORTED;
  // rows are copied in 16-byte pieces
  const uintptr_t align = reinterpret_cast<uintptr_t>(k_node) | reinterpret_cast<uintptr_t>(v_node) |
                          reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache);
  if (align & 15u) return TV_ERR_UNSUPPORTED;
  return launched(tv::launch_kv_commit(k_node, v_node, accepted_nodes, num_accepted, ctx_len,
                                       block_table, max_blocks_per_seq, num_blocks, B, N, Hkv, D,
                                       dtype, k_cache, v_cache, as_stream(stream)));
}

tv_status tree_draft_topk(const void* logits, int32_t B, int32_t L, int32_t V, int32_t K,
                          tv_dtype dtype, int32_t* cand_tokens, float* cand_logprob,
                          tv_stream stream) {
  if (!logits || !cand_tokens || !cand_logprob) return TV_ERR_NULL;
  if (B < 1 || L < 1 || V < 1 || K < 1) return TV_ERR_SHAPE;
  if (!dtype_ok(dtype)) return TV_ERR_UNSUPPORTED;
  if (L > TV_TREE_MAX_DEPTH || K > TV_TREE_MAX_TOPK || K > V) return TV_ERR_UNSUPPORTED;
  if (static_cast<long long>(B) * L > 0x7fffffffLL) return TV_ERR_UNSUPPORTED;
  return launched(tv::launch_draft_topk(logits, B, L, V, K, dtype, cand_tokens, cand_logprob,
                                        as_stream(stream)));
}

tv_status tree_build(const int32_t* cand_tokens, const float* cand_logprob, int32_t B, int32_t L,
                     int32_t K, int32_t N, int32_t w, int32_t* tokens, int32_t* parent,
                     int32_t* depth, float* score, int32_t* num_nodes, tv_stream stream) {
  if (!cand_tokens || !cand_logprob || !tokens || !parent || !depth || !num_nodes)
    return TV_ERR_NULL;
  if (B < 1 || L < 1 || K < 1 || N < 1 || w < 1) return TV_ERR_SHAPE;
  if (L > TV_TREE_MAX_DEPTH || K > TV_TREE_MAX_TOPK || N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
  return launched(tv::launch_tree_build(cand_tokens, cand_logprob, B, L, K, N, w, tokens, parent,
                                        depth, score, num_nodes, as_stream(stream)));
}

size_t tree_walk_accept_workspace_size(int32_t B, int32_t N) {
  if (B < 1 || N < 1) return 0;
  return static_cast<size_t>(B) * (N + 1) * sizeof(int32_t);
}

tv_status tree_walk_accept(const int32_t* tokens, const int32_t* parent, const void* logits,
                           int32_t B, int32_t N, int32_t V, tv_dtype dtype,
                           int32_t* accepted_tokens, int32_t* accepted_nodes,
                           int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                           tv_stream stream) {
  if (!tokens || !parent || !logits || !accepted_tokens || !accepted_nodes || !num_accepted)
    return TV_ERR_NULL;
  if (B < 1 || N < 1 || V < 1) return TV_ERR_SHAPE;
  if (!dtype_ok(dtype)) return TV_ERR_UNSUPPORTED;
  if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
  if (static_cast<long long>(B) * (N + 1) > 0x7fffffffLL) return TV_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < tree_walk_accept_workspace_size(B, N))
    return TV_ERR_WORKSPACE;
  return launched(tv::launch_walk(tokens, parent, logits, B, N, V, dtype, accepted_tokens,
                                  accepted_nodes, num_accepted, static_cast<int32_t*>(workspace),
                                  as_stream(stream)));
}

tv_status tree_walk_accept_noalloc(const int32_t* tokens, const int32_t* parent,
                                   const void* logits, int32_t B, int32_t N, int32_t V,
                                   tv_dtype dtype, int32_t* accepted_tokens,
                                   int32_t* accepted_nodes, int32_t* num_accepted,
                                   tv_stream stream) {
  if (!tokens || !parent || !logits || !accepted_tokens || !accepted_nodes || !num_accepted)
    return TV_ERR_NULL;
  if (B < 1 || N < 1 || V < 1) return TV_ERR_SHAPE;
  if (!dtype_ok(dtype)) return TV_ERR_UNSUPPORTED;
  if (N > TV_MAX_NODES) return TV_ERR_UNSUPPORTED;
  if (static_cast<long long>(B) * (N + 1) > TV_WALK_NOALLOC_MAX_ROWS) return TV_ERR_SCRATCH;
  return launched(tv::launch_walk_noalloc(tokens, parent, logits, B, N, V, dtype, accepted_tokens,
                                          accepted_nodes, num_accepted, as_stream(stream)));
}

}  // extern "C"
