// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tree_verify.h"

namespace tv {

// bf16 <-> fp32 (bf16 is carried as its 16 raw bits)
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// round to nearest, ties to even; NaN stays a (quiet) NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 64-bit lane shuffle as two 32-bit ones
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl(static_cast<uint32_t>(v), src, 64);
  uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// compute units of the current device (256 on an MI355X; that value also
// when no device can be queried, e.g. for a size query on a host without one)
int device_cus();

// XCDs (accelerator complex dies) of the current device, -1 when the runtime
// does not say, 0 without a device
int device_xcds();

// ---- launchers (one per kernel family); return the launch error
hipError_t launch_mask(const int32_t* parent, const int32_t* depth_in, const int32_t* ctx_len,
                       int B, int N, uint64_t* anc, int32_t* depth_out, int32_t* pos,
                       float* dense_bias, int32_t* status, hipStream_t stream);

hipError_t launch_gdn_commit(const void* k, const void* v, const float* alpha, const float* beta,
                             const float* S0, const int32_t* acc_nodes, const int32_t* num_acc,
                             int B, int N, int H, tv_dtype dtype, float* S_out,
                             hipStream_t stream);

hipError_t launch_kv_commit(const void* k_node, const void* v_node, const int32_t* acc_nodes,
                            const int32_t* num_acc, const int32_t* ctx_len, const int32_t* bt,
                            int max_blocks, int num_blocks, int B, int N, int Hkv, int D,
                            tv_dtype dtype, void* k_cache, void* v_cache, hipStream_t stream);

hipError_t launch_walk(const int32_t* tokens, const int32_t* parent, const void* logits, int B,
                       int N, int V, tv_dtype dtype, int32_t* acc_tok, int32_t* acc_node,
                       int32_t* num_acc, int32_t* argmax_ws, hipStream_t stream);

hipError_t launch_walk_noalloc(const int32_t* tokens, const int32_t* parent, const void* logits,
                               int B, int N, int V, tv_dtype dtype, int32_t* acc_tok,
                               int32_t* acc_node, int32_t* num_acc, hipStream_t stream);

hipError_t launch_draft_topk(const void* logits, int B, int L, int V, int K, tv_dtype dtype,
                             int32_t* cand_tok, float* cand_lp, hipStream_t stream);

hipError_t launch_tree_build(const int32_t* cand_tok, const float* cand_lp, int B, int L, int K,
                             int N, int w, int32_t* tokens, int32_t* parent, int32_t* depth,
                             float* score, int32_t* num_nodes, hipStream_t stream);

struct AttnPlan {
  int G;            // query heads per kv head
  int rows;         // G * N query rows per (sequence, kv head)
  int row_groups;   // ceil(rows / rows per workgroup)
  int nsplit;       // maximum context splits per (sequence, kv head)
  int split_tokens; // nominal tokens per split (multiple of the key tile)
  int stream_wg;    // > 0: stream layout over this many workgroups, no splits
  int stream_pm;    // thousandths of a CU pair's tiles for its first workgroup
  int stream_xm;    // thousandths of the average share for workgroups on even XCDs
  size_t ws_bytes;  // partials
};

AttnPlan attn_plan(int B, int N, int Hq, int Hkv, int D, int max_ctx_len, int window);

hipError_t launch_attn(const AttnPlan& plan, const void* q, const void* k_node,
                       const void* v_node, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int max_blocks, int num_blocks,
                       const int32_t* ctx_len, int max_ctx_len, const uint64_t* anc,
                       const int32_t* pos, int B, int N, int Hq, int Hkv, int D, int window,
                       float scale, tv_dtype dtype, tv_dtype out_dtype, void* out, void* ws,
                       hipStream_t stream);

hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                      int H, int Dk, int Dv, tv_dtype dtype, tv_dtype out_dtype, void* out,
                      hipStream_t stream);

}  // namespace tv
