// Ancestor-or-self mask, depth and position ids of a flattened draft tree.
//
// Serve-integration spec, section "2. Verify: tree attention mask": a node
// sees only its ancestors and itself among the draft nodes, and its position
// id is ctx_len - 1 + depth.  One wave64 per tree, lane = node: the ancestor
// word of a node is its own bit or-ed with its parent's word, which the wave
// settles level by level (at most depth rounds) through lane shuffles.
#include "tv_internal.h"

namespace tv {

__global__ __launch_bounds__(64) void mask_kernel(const int32_t* __restrict__ parent,
                                                  const int32_t* __restrict__ depth_in,
                                                  const int32_t* __restrict__ ctx_len, int N,
                                                  uint64_t* __restrict__ anc,
                                                  int32_t* __restrict__ depth_out,
                                                  int32_t* __restrict__ pos,
                                                  float* __restrict__ dense_bias,
                                                  int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const bool act = t < N;
  const size_t base = static_cast<size_t>(b) * N;

  int p = act ? parent[base + t] : -1;
  const bool bad = act && !(p >= -1 && p < t);
  const bool any_bad = __ballot(bad) != 0ull;
  const int ctx = ctx_len[b];
  const uint64_t self = act ? (1ull << t) : 0ull;

  uint64_t a = self;
  if (any_bad) {
    p = -1;  // star fallback: every node sees only itself
  } else {
    // a[t] = bit(t) | a[parent(t)]; each round settles one more tree level
    for (int round = 0; round < N; ++round) {
      uint64_t pa = shfl_u64(a, p >= 0 ? p : t);
      uint64_t na = self | (p >= 0 ? pa : 0ull);
      bool changed = na != a;
      a = na;
      if (__ballot(act && changed) == 0ull) break;
    }
  }
  const int d = __popcll(a);

  int st = TV_TREE_OK;
  if (any_bad) {
    st = TV_TREE_BAD_PARENT;
  } else {
    bool dbad = act && depth_in != nullptr && depth_in[base + t] != d;
    if (__ballot(dbad) != 0ull) st = TV_TREE_BAD_DEPTH;
    else if (ctx < 1) st = TV_TREE_BAD_CTX;
  }

  if (act) {
    anc[base + t] = a;
    depth_out[base + t] = d;
    pos[base + t] = ctx - 1 + d;
  }
  if (t == 0) status[b] = st;

  if (dense_bias != nullptr) {
    // row r of this tree: lanes sweep the columns so that stores coalesce
    float* rowp = dense_bias + base * N;
    for (int r = 0; r < N; ++r) {
      uint64_t ar = shfl_u64(a, r);
      if (act) rowp[static_cast<size_t>(r) * N + t] = ((ar >> t) & 1ull) ? 0.0f : -INFINITY;
    }
  }
}

hipError_t launch_mask(const int32_t* parent, const int32_t* depth_in, const int32_t* ctx_len,
                       int B, int N, uint64_t* anc, int32_t* depth_out, int32_t* pos,
                       float* dense_bias, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(mask_kernel, dim3(B), dim3(64), 0, stream, parent, depth_in, ctx_len, N,
                     anc, depth_out, pos, dense_bias, status);
  return hipGetLastError();
}

}  // namespace tv
