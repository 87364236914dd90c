// Draft-tree construction on the GPU: the step before verification.
//
// DDTree validation post, section "The Failed First Attempt": the tree grows
// best-first from a priority queue on cumulative log-probability, from the
// top-k tokens of the first position as roots; a popped node joins the tree
// and its sibling and child go back on the queue, up to a node budget and a
// maximum depth.  DFlash-TfM summary, section "2. Boomconstructie": the top-w
// candidates leave the queue together and are expanded together, so a budget
// of n takes ceil(n / w) rounds.  The draft distribution is factorised per
// depth: one list of K candidates per depth, the same under every parent.
//
// Two kernels.  draft_topk_kernel: per (sequence, depth) row of draft logits,
// the log-sum-exp over the vocabulary and the K largest logits (ties to the
// lower token id), in one pass (an HBM stream).  tree_build_kernel: one wave
// per sequence runs the queue in LDS; a candidate's push counter is its slot
// in the pool, so "equal scores in push order" is "equal scores, lower slot".
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kTopkThreads = 512;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kKMax = TV_TREE_MAX_TOPK;  // per-thread candidate list length

// order of the top-k selection: larger value first, then lower index
__device__ __forceinline__ bool cand_before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// the wave's best (value, index) pair and the lane that holds it
__device__ __forceinline__ void wave_best(float& v, int& i, int& lane_of) {
  lane_of = static_cast<int>(threadIdx.x & 63);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    const int ol = __shfl_xor(lane_of, off, 64);
    if (cand_before(ov, oi, v, i)) {
      v = ov;
      i = oi;
      lane_of = ol;
    }
  }
}

template <typename T>
__device__ __forceinline__ float elem(const T* p, size_t i) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  else return p[i];
}

// Row r = (sequence, depth) of V logits: K candidates and their log-softmax
// values.  Each thread scans 16-byte chunks c = tid, tid + 512, ... keeping a
// running (max, sum of exp2).  Each wave keeps one sorted list of its K best
// (lane k < K holds entry k): an element is a candidate only if it beats the
// list's last entry, which the whole wave knows, so after the first few
// chunks a chunk costs a compare and a ballot per element; the rare
// candidates enter one at a time by a lane-parallel insertion.  The four
// waves' lists merge at the end.
template <typename T>
__global__ __launch_bounds__(kTopkThreads) void draft_topk_kernel(const T* __restrict__ logits,
                                                                  int V, int K,
                                                                  int32_t* __restrict__ cand_tok,
                                                                  float* __restrict__ cand_lp) {
  constexpr float kLog2e = 1.4426950408889634f;
  const size_t row = blockIdx.x;
  const T* p = logits + row * static_cast<size_t>(V);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  float wv = -INFINITY;  // this lane's entry of the wave list (lanes < K)
  int wi = 0x7fffffff;
  float thr = -INFINITY;  // the list's entry K - 1 (wave-uniform)
  int thr_i = 0x7fffffff;
  auto consider = [&](float v, int idx) __attribute__((always_inline)) {
    uint64_t mask = __ballot(cand_before(v, idx, thr, thr_i));
    while (mask != 0ull) {
      const int src = __ffsll(static_cast<unsigned long long>(mask)) - 1;
      mask &= mask - 1ull;
      const float cv = __shfl(v, src, 64);
      const int ci = __shfl(idx, src, 64);
      if (!cand_before(cv, ci, thr, thr_i)) continue;  // the list moved on
      // entries after the insertion point move down one lane
      const uint64_t worse = __ballot(lane < K && cand_before(cv, ci, wv, wi));
      const int pos = __ffsll(static_cast<unsigned long long>(worse)) - 1;
      const float up_v = __shfl_up(wv, 1, 64);
      const int up_i = __shfl_up(wi, 1, 64);
      if (lane < K && lane >= pos) {
        wv = lane == pos ? cv : up_v;
        wi = lane == pos ? ci : up_i;
      }
      thr = __shfl(wv, K - 1, 64);
      thr_i = __shfl(wi, K - 1, 64);
    }
  };
  float m = -INFINITY, s = 0.0f;  // running max and sum of exp2((x - m) log2 e)

  constexpr int E = 16 / static_cast<int>(sizeof(T));  // elements per chunk
  const bool vec = ((static_cast<size_t>(V) * sizeof(T)) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  const int nchunk = vec ? V / E : 0;
  // one chunk: the running max and sum absorb it, and its elements are offered
  // to the wave list.  Called by the whole wave (the list lives in its first K
  // lanes); a lane without a chunk offers nothing.
  auto absorb = [&](const u32x4_t raw, int c, bool valid) __attribute__((always_inline)) {
    float x[E];
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {raw[0], raw[1], raw[2], raw[3]};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    } else {
      x[0] = __uint_as_float(raw[0]);
      x[1] = __uint_as_float(raw[1]);
      x[2] = __uint_as_float(raw[2]);
      x[3] = __uint_as_float(raw[3]);
    }
    float cm = x[0];
#pragma unroll
    for (int k = 1; k < E; ++k) cm = fmaxf(cm, x[k]);
    if (valid) {
      const float nm = fmaxf(m, cm);
      float add = 0.0f;
#pragma unroll
      for (int k = 0; k < E; ++k) add += __builtin_amdgcn_exp2f((x[k] - nm) * kLog2e);
      s = (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((m - nm) * kLog2e)) + add;
      m = nm;
    }
    if (__ballot(valid && cm >= thr) != 0ull) {
#pragma unroll
      for (int k = 0; k < E; ++k) consider(valid ? x[k] : -INFINITY, valid ? c * E + k : 0x7fffffff);
    }
  };
  // kU loads in flight per thread, then their chunks; the loop bounds are
  // wave-uniform (cw = the wave's first chunk of a pass)
  constexpr int kU = 8;
  const u32x4_t* pc = reinterpret_cast<const u32x4_t*>(p);
  int cw = wave * 64;
  for (; cw + 63 + (kU - 1) * kTopkThreads < nchunk; cw += kU * kTopkThreads) {
    u32x4_t r[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) r[u] = __builtin_nontemporal_load(pc + cw + lane + u * kTopkThreads);
#pragma unroll
    for (int u = 0; u < kU; ++u) absorb(r[u], cw + lane + u * kTopkThreads, true);
  }
  for (; cw < nchunk; cw += kTopkThreads) {
    const int c = cw + lane;
    const bool ok = c < nchunk;
    const u32x4_t r = ok ? __builtin_nontemporal_load(pc + c) : u32x4_t{0u, 0u, 0u, 0u};
    absorb(r, c, ok);
  }
  // elements past the last whole chunk (or every element without 16-byte
  // rows); the loop runs while any lane of the wave has one
  for (int v0 = nchunk * E + (tid & ~63); v0 < V; v0 += kTopkThreads) {
    const int v = v0 + lane;
    const float x = v < V ? elem(p, v) : -INFINITY;
    if (v < V) {
      const float nm = fmaxf(m, x);
      s = (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((m - nm) * kLog2e)) +
          __builtin_amdgcn_exp2f((x - nm) * kLog2e);
      m = nm;
    }
    consider(x, v < V ? v : 0x7fffffff);
  }

  // log-sum-exp over the workgroup
  __shared__ float s_m[kTopkThreads / 64], s_s[kTopkThreads / 64];
  __shared__ float s_lv[kTopkThreads / 64][kKMax];
  __shared__ int s_li[kTopkThreads / 64][kKMax];
  float wm = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off, 64));
  float ws = m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((m - wm) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off, 64);
  if (lane < K) {
    s_lv[wave][lane] = wv;
    s_li[wave][lane] = wi;
  }
  if (lane == 0) {
    s_m[wave] = wm;
    s_s[wave] = ws;
  }
  __syncthreads();
  if (wave != 0) return;
  float gm = -INFINITY;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) gm = fmaxf(gm, s_m[w]);
  float gs = 0.0f;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w)
    gs += s_m[w] == -INFINITY ? 0.0f : s_s[w] * __builtin_amdgcn_exp2f((s_m[w] - gm) * kLog2e);
  const float lse = gm + __builtin_amdgcn_logf(gs) * 0.6931471805599453f;
  // merge the waves' lists: lane j holds entries j and j + 64 of the
  // concatenated lists (entry e = entry e % K of wave e / K), offering the
  // better of the two it still has
  constexpr int nw = kTopkThreads / 64;
  static_assert(nw * kKMax <= 128, "two merge entries per lane");
  float ev[2];
  int ei[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = lane + 64 * q;
    ev[q] = e < nw * K ? s_lv[e / K][e % K] : -INFINITY;
    ei[q] = e < nw * K ? s_li[e / K][e % K] : 0x7fffffff;
  }
  for (int k = 0; k < K; ++k) {
    const bool second = cand_before(ev[1], ei[1], ev[0], ei[0]);
    float v = second ? ev[1] : ev[0];
    int i = second ? ei[1] : ei[0];
    int owner;
    wave_best(v, i, owner);
    if (lane == owner) {
      if (second) {
        ev[1] = -INFINITY;
        ei[1] = 0x7fffffff;
      } else {
        ev[0] = -INFINITY;
        ei[0] = 0x7fffffff;
      }
    }
    if (lane == 0) {
      cand_tok[row * K + k] = i;
      cand_lp[row * K + k] = v - lse;
    }
  }
}

// Pool of queued candidates (slot = push counter) and popped nodes, in LDS.
constexpr int kPoolMax = TV_TREE_MAX_TOPK + 2 * TV_MAX_NODES;

__device__ __forceinline__ int meta_pack(int depth, int rank, int parent) {
  return ((parent + 1) << 10) | (depth << 5) | rank;
}
__device__ __forceinline__ int meta_depth(int m) { return (m >> 5) & 31; }
__device__ __forceinline__ int meta_rank(int m) { return m & 31; }
__device__ __forceinline__ int meta_parent(int m) { return (m >> 10) - 1; }

// One wave per sequence.  Rounds pop min(w, budget left, queued) candidates
// (best score first, equal scores by lower slot), then push, for each popped
// node in pop order, its next sibling (depth >= 2) and its first child (below
// the maximum depth).  The popped nodes are then flattened by depth (stable)
// and their parents renumbered.
__global__ __launch_bounds__(64) void tree_build_kernel(const int32_t* __restrict__ cand_tok,
                                                        const float* __restrict__ cand_lp, int L,
                                                        int K, int N, int w,
                                                        int32_t* __restrict__ tokens,
                                                        int32_t* __restrict__ parent,
                                                        int32_t* __restrict__ depth,
                                                        float* __restrict__ score,
                                                        int32_t* __restrict__ num_nodes) {
  __shared__ float p_score[kPoolMax];
  __shared__ int p_meta[kPoolMax];
  __shared__ float n_score[TV_MAX_NODES];
  __shared__ int n_meta[TV_MAX_NODES];
  __shared__ float s_lp[TV_TREE_MAX_DEPTH * TV_TREE_MAX_TOPK];
  __shared__ int s_new[TV_MAX_NODES];
  const int b = blockIdx.x, lane = threadIdx.x;
  const float* lp_b = cand_lp + static_cast<size_t>(b) * L * K;
  for (int e = lane; e < L * K; e += 64) s_lp[e] = lp_b[e];
  for (int e = lane; e < kPoolMax; e += 64) p_score[e] = -INFINITY;
  __syncthreads();
  // the roots: the K depth-1 candidates in rank order (slots 0 .. K - 1)
  for (int r = lane; r < K; r += 64) {
    p_score[r] = s_lp[r];
    p_meta[r] = meta_pack(1, r, -1);
  }
  int pushed = K;  // slots used (= pushes so far)
  int queued = K;  // live candidates
  int n = 0;       // popped nodes
  __syncthreads();
  while (n < N && queued > 0) {
    const int take = min(min(w, N - n), queued);
    for (int t = 0; t < take; ++t) {
      // best live slot: larger score, then lower slot (empty slots are -inf
      // and marked by a meta of -1)
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int e = lane; e < pushed; e += 64) {
        const float v = p_score[e];
        if (p_meta[e] >= 0 && cand_before(v, e, bv, bi)) {
          bv = v;
          bi = e;
        }
      }
      int owner;
      wave_best(bv, bi, owner);
      if (lane == 0) {
        n_score[n + t] = p_score[bi];
        n_meta[n + t] = p_meta[bi];
        p_meta[bi] = -1;
      }
      __syncthreads();
    }
    if (lane == 0) {
      for (int t = 0; t < take; ++t) {
        const int me = n + t;
        const int m = n_meta[me];
        const int d = meta_depth(m), r = meta_rank(m), par = meta_parent(m);
        if (d >= 2 && r + 1 < K) {
          p_score[pushed] = n_score[par] + s_lp[(d - 1) * K + r + 1];
          p_meta[pushed] = meta_pack(d, r + 1, par);
          ++pushed;
          ++queued;
        }
        if (d < L) {
          p_score[pushed] = n_score[me] + s_lp[d * K];
          p_meta[pushed] = meta_pack(d + 1, 0, me);
          ++pushed;
          ++queued;
        }
      }
    }
    n += take;
    queued -= take;
    pushed = __shfl(pushed, 0, 64);
    queued = __shfl(queued, 0, 64);
    __syncthreads();
  }

  // flatten by depth, stable: new index = nodes of smaller depth + nodes of
  // the same depth popped earlier
  for (int i = lane; i < n; i += 64) {
    const int di = meta_depth(n_meta[i]);
    int pos = 0;
    for (int j = 0; j < n; ++j) {
      const int dj = meta_depth(n_meta[j]);
      pos += (dj < di) || (dj == di && j < i);
    }
    s_new[i] = pos;
  }
  __syncthreads();
  const size_t ob = static_cast<size_t>(b) * N;
  const int32_t* tok_b = cand_tok + static_cast<size_t>(b) * L * K;
  for (int i = lane; i < N; i += 64) {
    if (i < n) {
      const int m = n_meta[i];
      const int d = meta_depth(m), r = meta_rank(m), par = meta_parent(m);
      const int o = s_new[i];
      tokens[ob + o] = tok_b[(d - 1) * K + r];
      parent[ob + o] = par < 0 ? -1 : s_new[par];
      depth[ob + o] = d;
      if (score != nullptr) score[ob + o] = n_score[i];
    } else {
      tokens[ob + i] = -1;
      parent[ob + i] = -1;
      depth[ob + i] = 0;
      if (score != nullptr) score[ob + i] = -INFINITY;
    }
  }
  if (lane == 0) num_nodes[b] = n;
}

}  // namespace

hipError_t launch_draft_topk(const void* logits, int B, int L, int V, int K, tv_dtype dtype,
                             int32_t* cand_tok, float* cand_lp, hipStream_t stream) {
  const unsigned rows = static_cast<unsigned>(B) * static_cast<unsigned>(L);
  if (dtype == TV_BF16)
    hipLaunchKernelGGL(draft_topk_kernel<uint16_t>, dim3(rows), dim3(kTopkThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), V, K, cand_tok, cand_lp);
  else
    hipLaunchKernelGGL(draft_topk_kernel<float>, dim3(rows), dim3(kTopkThreads), 0, stream,
                       static_cast<const float*>(logits), V, K, cand_tok, cand_lp);
  return hipGetLastError();
}

hipError_t launch_tree_build(const int32_t* cand_tok, const float* cand_lp, int B, int L, int K,
                             int N, int w, int32_t* tokens, int32_t* parent, int32_t* depth,
                             float* score, int32_t* num_nodes, hipStream_t stream) {
  hipLaunchKernelGGL(tree_build_kernel, dim3(B), dim3(64), 0, stream, cand_tok, cand_lp, L, K, N, w,
                     tokens, parent, depth, score, num_nodes);
  return hipGetLastError();
}

}  // namespace tv
