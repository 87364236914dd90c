// Ancestor-or-self mask, depth and position ids of a flattened draft tree.
//
// Serve-integration spec, section "2. Verify: tree attention mask": a node
// sees only its ancestors and itself among the draft nodes, and its position
// id is ctx_len - 1 + depth.  One workgroup per tree, thread = node.  The
// ancestor set is built by pointer jumping: each node keeps the set of the
// path from itself up to (not including) a jump target, and each round joins
// the target's set and moves the target to the target's target, so the path
// covered doubles per round and ceil(log2 N) rounds settle any tree (a chain
// of 128 nodes takes 7).  Sets are ceil(N / 64) 64-bit words, node j being
// bit j % 64 of word j / 64.
#include "tv_internal.h"

namespace tv {

constexpr int kMaskWords = (TV_MAX_NODES + 63) / 64;

__global__ __launch_bounds__(TV_MAX_NODES) void mask_kernel(const int32_t* __restrict__ parent,
                                                            const int32_t* __restrict__ depth_in,
                                                            const int32_t* __restrict__ ctx_len,
                                                            int N, uint64_t* __restrict__ anc,
                                                            int32_t* __restrict__ depth_out,
                                                            int32_t* __restrict__ pos,
                                                            float* __restrict__ dense_bias,
                                                            int32_t* __restrict__ status) {
  __shared__ uint64_t s_set[TV_MAX_NODES][kMaskWords];
  __shared__ int s_jump[TV_MAX_NODES];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int nw = (N + 63) / 64;
  const bool act = t < N;
  const size_t base = static_cast<size_t>(b) * N;

  int p = act ? parent[base + t] : -1;
  const int ctx = ctx_len[b];
  const int din = (act && depth_in != nullptr) ? depth_in[base + t] : 0;
  const bool bad = act && !(p >= -1 && p < t);
  const bool any_bad = __syncthreads_or(bad) != 0;
  if (any_bad) p = -1;  // star fallback: every node sees only itself

  uint64_t a[kMaskWords];
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) a[w] = (act && (t >> 6) == w) ? (1ull << (t & 63)) : 0ull;
  int j = p;
  // invariant: a = the nodes from t up to, not including, j (-1: the root)
  while (__syncthreads_or(j >= 0)) {
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) s_set[t][w] = a[w];
    s_jump[t] = j;
    __syncthreads();
    if (j >= 0) {
#pragma unroll
      for (int w = 0; w < kMaskWords; ++w) a[w] |= s_set[j][w];
      j = s_jump[j];
    }
    __syncthreads();  // the next round overwrites the tables
  }
  int d = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) d += __popcll(a[w]);

  int st = TV_TREE_OK;
  if (any_bad) {
    st = TV_TREE_BAD_PARENT;
  } else if (__syncthreads_or(act && depth_in != nullptr && din != d)) {
    st = TV_TREE_BAD_DEPTH;
  } else if (ctx < 1) {
    st = TV_TREE_BAD_CTX;
  }

  if (act) {
    for (int w = 0; w < nw; ++w) anc[(base + t) * nw + w] = a[w];
    depth_out[base + t] = d;
    pos[base + t] = ctx - 1 + d;
  }
  if (t == 0) status[b] = st;

  if (dense_bias != nullptr) {
#pragma unroll
    for (int w = 0; w < kMaskWords; ++w) s_set[t][w] = a[w];
    __syncthreads();
    // row r of this tree: threads sweep the columns so that stores coalesce
    float* rowp = dense_bias + base * N;
    for (int e = t; e < N * N; e += blockDim.x) {
      const int r = e / N, c = e % N;
      rowp[e] = ((s_set[r][c >> 6] >> (c & 63)) & 1ull) ? 0.0f : -INFINITY;
    }
  }
}

hipError_t launch_mask(const int32_t* parent, const int32_t* depth_in, const int32_t* ctx_len,
                       int B, int N, uint64_t* anc, int32_t* depth_out, int32_t* pos,
                       float* dense_bias, int32_t* status, hipStream_t stream) {
  const int threads = 64 * ((N + 63) / 64);
  hipLaunchKernelGGL(mask_kernel, dim3(B), dim3(threads), 0, stream, parent, depth_in, ctx_len, N,
                     anc, depth_out, pos, dense_bias, status);
  return hipGetLastError();
}

}  // namespace tv
