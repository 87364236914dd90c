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

// One workgroup per (sequence, head): thread t holds columns 4 (t % 32) .. +3
// of rows 16 (t / 32) .. +15 of the 128 x 128 state, in registers, so that
// the state moves in 16-byte pieces.  The accepted nodes' keys, values and
// gates are staged in LDS, 64 steps at a time (one batch of loads); each step forms
// u = k^T S (eight partial sums per column, combined through LDS) and applies
// S <- alpha S + k (beta (v - alpha u))^T, which is the recurrence written
// out.  S0 and S_out may be the same buffer: each workgroup reads its whole
// state before writing it.
constexpr int kGD = 128;  // Dk = Dv

constexpr int kChunk = 64;  // accepted steps staged in LDS at a time

template <typename T>
__global__ __launch_bounds__(256) void gdn_commit_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* S0, const int32_t* __restrict__ acc_nodes,
    const int32_t* __restrict__ num_acc, int N, int H, float* S_out) {
  __shared__ __align__(16) float s_kv[kChunk][2 * kGD];  // [step][k | v]
  __shared__ float2 s_ab[kChunk];                        // (alpha, beta) per step
  __shared__ __align__(16) float s_u[8][kGD];            // partial k^T S per row group
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const int cg = tid % 32, rg = tid / 32;  // columns 4 cg .. 4 cg + 3, rows 16 rg .. 16 rg + 15
  const int a = min(max(num_acc[b], 0), N);
  const size_t sbase = (static_cast<size_t>(b) * H + h) * kGD * kGD;

  float4 S[16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    S[r] = *reinterpret_cast<const float4*>(S0 + sbase + static_cast<size_t>(16 * rg + r) * kGD + 4 * cg);
  constexpr int kPer = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte piece
  constexpr int kPieces = kGD / kPer;                      // pieces per row
  for (int c0 = 0; c0 < a; c0 += kChunk) {
    const int na = min(kChunk, a - c0);
    // keys and values of the chunk's accepted steps, 16 bytes per load
    for (int e = tid; e < na * 2 * kPieces; e += 256) {
      const int st = e / (2 * kPieces), c = e % (2 * kPieces);
      const int node = min(max(acc_nodes[static_cast<size_t>(b) * N + c0 + st], 0), N - 1);
      const size_t row = (static_cast<size_t>(b) * N + node) * H + h;
      const bool isv = c >= kPieces;
      const int piece = isv ? c - kPieces : c;
      const uint4 raw = *reinterpret_cast<const uint4*>((isv ? v : k) + row * kGD + piece * kPer);
      float* dst = &s_kv[st][(isv ? kGD : 0) + piece * kPer];
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[2 * i] = bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffffu));
          dst[2 * i + 1] = bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
        }
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y),
                                                      __uint_as_float(raw.z), __uint_as_float(raw.w));
      }
    }
    if (tid < na) {
      const int node = min(max(acc_nodes[static_cast<size_t>(b) * N + c0 + tid], 0), N - 1);
      const size_t g = (static_cast<size_t>(b) * N + node) * H + h;
      s_ab[tid] = make_float2(alpha[g], beta[g]);
    }
    __syncthreads();

    for (int st = 0; st < na; ++st) {
      float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kr = s_kv[st][16 * rg + r];
        p.x += kr * S[r].x;
        p.y += kr * S[r].y;
        p.z += kr * S[r].z;
        p.w += kr * S[r].w;
      }
      *reinterpret_cast<float4*>(&s_u[rg][4 * cg]) = p;
      __syncthreads();
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 q = *reinterpret_cast<const float4*>(&s_u[i][4 * cg]);
        u.x += q.x;
        u.y += q.y;
        u.z += q.z;
        u.w += q.w;
      }
      const float al = s_ab[st].x, be = s_ab[st].y;
      const float4 vv = *reinterpret_cast<const float4*>(&s_kv[st][kGD + 4 * cg]);
      const float4 wv = make_float4(be * (vv.x - al * u.x), be * (vv.y - al * u.y),
                                    be * (vv.z - al * u.z), be * (vv.w - al * u.w));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kr = s_kv[st][16 * rg + r];
        S[r].x = al * S[r].x + kr * wv.x;
        S[r].y = al * S[r].y + kr * wv.y;
        S[r].z = al * S[r].z + kr * wv.z;
        S[r].w = al * S[r].w + kr * wv.w;
      }
      __syncthreads();  // s_u (and, after the last step, the staged chunk) is rewritten next
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *reinterpret_cast<float4*>(S_out + sbase + static_cast<size_t>(16 * rg + r) * kGD + 4 * cg) = S[r];
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
  // the three loads go out together
  const int na = num_acc[b];
  const int node = acc_nodes[static_cast<size_t>(b) * N + s];
  const int p = ctx_len[b] + s;
  if (s >= na) return;
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
