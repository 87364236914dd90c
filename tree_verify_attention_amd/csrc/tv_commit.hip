// Commits after the walk: the accepted path's keys and values into the paged
// cache, and the Gated DeltaNet state advanced over the accepted nodes.
//
// Serve-integration spec, layout contract and "3. Rejection sampler: tree
// walk": accepted node s (depth s + 1) has position id ctx_len - 1 + depth =
// ctx_len + s, one past the last accepted token; its key and value rows come
// from the verify pass.  DFlash-TfM summary, section "3. Rollback-vrije
// Boom-verificatie voor GDN": the state is published only once the accepted
// branch is known, by the recurrence S_t = alpha_t (I - beta_t k_t k_t^T)
// S_{t-1} + beta_t k_t v_t^T along it.
#include "tv_internal.h"

namespace tv {

namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(x);
  else return x;
}

// One workgroup per (sequence, head): thread t holds column j = t % 128 of
// the 128 x 128 state, rows 64 (t / 128) .. +63, in registers.  The accepted
// nodes' keys, values and gates are staged in LDS first (one batch of loads);
// each step forms u = k^T S (two half sums per column, combined through LDS)
// and applies S <- alpha S + k (beta (v - alpha u))^T, which is the
// recurrence written out.  S0 and S_out may be the same buffer: each
// workgroup reads its whole state before writing it.
constexpr int kGD = 128;  // Dk = Dv

template <typename T>
__global__ __launch_bounds__(256) void gdn_commit_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* S0, const int32_t* __restrict__ acc_nodes,
    const int32_t* __restrict__ num_acc, int N, int H, float* S_out) {
  __shared__ float s_kv[TV_MAX_NODES][2 * kGD];  // [step][k | v]
  __shared__ float2 s_ab[TV_MAX_NODES];          // (alpha, beta) per step
  __shared__ float s_u[2][kGD];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const int j = tid % kGD, half = tid / kGD;
  const int a = min(max(num_acc[b], 0), N);
  const size_t sbase = (static_cast<size_t>(b) * H + h) * kGD * kGD;

  float S[kGD / 2];
#pragma unroll
  for (int r = 0; r < kGD / 2; ++r) S[r] = S0[sbase + static_cast<size_t>(half * 64 + r) * kGD + j];
  for (int e = tid; e < a * 2 * kGD; e += 256) {
    const int s = e / (2 * kGD), c = e % (2 * kGD);
    const int node = min(max(acc_nodes[static_cast<size_t>(b) * N + s], 0), N - 1);
    const size_t row = (static_cast<size_t>(b) * N + node) * H + h;
    s_kv[s][c] = c < kGD ? to_f32(k[row * kGD + c]) : to_f32(v[row * kGD + c - kGD]);
  }
  if (tid < a) {
    const int node = min(max(acc_nodes[static_cast<size_t>(b) * N + tid], 0), N - 1);
    const size_t g = (static_cast<size_t>(b) * N + node) * H + h;
    s_ab[tid] = make_float2(alpha[g], beta[g]);
  }
  __syncthreads();

  for (int s = 0; s < a; ++s) {
    float p = 0.0f;
#pragma unroll
    for (int r = 0; r < kGD / 2; ++r) p += s_kv[s][half * 64 + r] * S[r];
    s_u[half][j] = p;
    __syncthreads();
    const float u = s_u[0][j] + s_u[1][j];
    const float al = s_ab[s].x, be = s_ab[s].y;
    const float w = be * (s_kv[s][kGD + j] - al * u);
#pragma unroll
    for (int r = 0; r < kGD / 2; ++r) S[r] = al * S[r] + s_kv[s][half * 64 + r] * w;
    __syncthreads();  // s_u is rewritten by the next step
  }
#pragma unroll
  for (int r = 0; r < kGD / 2; ++r) S_out[sbase + static_cast<size_t>(half * 64 + r) * kGD + j] = S[r];
}

// One workgroup per (sequence, accepted slot s): copies the node's key and
// value rows of every kv head into the page slot of position ctx_len + s, in
// 16-byte pieces.  Slots past num_accepted, node indices outside [0, N),
// negative positions and pages outside the table or the pool are skipped.
template <typename T>
__global__ __launch_bounds__(256) void kv_commit_kernel(
    const T* __restrict__ k_node, const T* __restrict__ v_node,
    const int32_t* __restrict__ acc_nodes, const int32_t* __restrict__ num_acc,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ bt, int max_blocks,
    int num_blocks, int N, int Hkv, int D, T* __restrict__ k_cache, T* __restrict__ v_cache) {
  const int b = blockIdx.x / N, s = blockIdx.x % N;
  if (s >= num_acc[b]) return;
  const int node = acc_nodes[static_cast<size_t>(b) * N + s];
  const int p = ctx_len[b] + s;
  if (node < 0 || node >= N || p < 0 || (p >> 4) >= max_blocks) return;
  const int page = bt[static_cast<size_t>(b) * max_blocks + (p >> 4)];
  if (page < 0 || page >= num_blocks) return;
  const int pieces = D * static_cast<int>(sizeof(T)) / 16;  // per kv head row
  for (int e = threadIdx.x; e < 2 * Hkv * pieces; e += 256) {
    const int which = e / (Hkv * pieces);  // 0: keys, 1: values
    const int g = (e / pieces) % Hkv, c = e % pieces;
    const uint4* src = reinterpret_cast<const uint4*>(
        (which ? v_node : k_node) + ((static_cast<size_t>(b) * N + node) * Hkv + g) * D);
    uint4* dst = reinterpret_cast<uint4*>(
        (which ? v_cache : k_cache) + ((static_cast<size_t>(page) * Hkv + g) * 16 + (p & 15)) * D);
    dst[c] = src[c];
  }
}

}  // namespace

hipError_t launch_gdn_commit(const void* k, const void* v, const float* alpha, const float* beta,
                             const float* S0, const int32_t* acc_nodes, const int32_t* num_acc,
                             int B, int N, int H, tv_dtype dtype, float* S_out,
                             hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(B) * H), block(256);
  if (dtype == TV_BF16)
    hipLaunchKernelGGL(gdn_commit_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), alpha,
                       beta, S0, acc_nodes, num_acc, N, H, S_out);
  else
    hipLaunchKernelGGL(gdn_commit_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(k), static_cast<const float*>(v), alpha, beta,
                       S0, acc_nodes, num_acc, N, H, S_out);
  return hipGetLastError();
}

hipError_t launch_kv_commit(const void* k_node, const void* v_node, const int32_t* acc_nodes,
                            const int32_t* num_acc, const int32_t* ctx_len, const int32_t* bt,
                            int max_blocks, int num_blocks, int B, int N, int Hkv, int D,
                            tv_dtype dtype, void* k_cache, void* v_cache, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(B) * N), block(256);
  if (dtype == TV_BF16)
    hipLaunchKernelGGL(kv_commit_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(k_node), static_cast<const uint16_t*>(v_node),
                       acc_nodes, num_acc, ctx_len, bt, max_blocks, num_blocks, N, Hkv, D,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache));
  else
    hipLaunchKernelGGL(kv_commit_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(k_node), static_cast<const float*>(v_node),
                       acc_nodes, num_acc, ctx_len, bt, max_blocks, num_blocks, N, Hkv, D,
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache));
  return hipGetLastError();
}

}  // namespace tv
