// Gated DeltaNet over a draft tree, with no state written.
//
// DFlash-TfM summary ("Trees from Marginals"), section "3. Rollback-vrije
// Boom-verificatie voor GDN": the recurrence S_t = alpha_t (I - beta_t k_t
// k_t^T) S_parent + beta_t k_t v_t^T is evaluated for every node at once as a
// masked triangular solve over the ancestor interaction matrices.  Written
// out (gamma_t = product of alpha over t's root path, t included, and
// r(t, i) = gamma_t / gamma_i = product of alpha strictly below i down to t):
//
//   X[t, i] = beta_t r(t, i) k_t.k_i      i a strict ancestor of t
//   Y[t, i] = r(t, i) q_t.k_i             i an ancestor of t or t itself
//   (I + X) U = beta (V - gamma (K S0))   unit lower-triangular in node order
//   O = gamma (Q S0) + Y U                o_t = S_t^T q_t
//
// The section's (I + X) U = beta V carries the committed-state term in the
// same system.  Node t depends only on rows of smaller depth, so the solve
// runs level by level over depth.  Workgroup = (sequence, head, 32 output
// columns): the columns of U and O are independent, so the state S0 is read
// once in total while the (small) Gram terms are recomputed per column block.
// All arithmetic is fp32.
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kDk = 128;
constexpr int kCB = 32;  // output columns per workgroup
constexpr int kThreads = 256;

__device__ __forceinline__ float load_f(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_f(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store_f(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_f(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

size_t gdn_lds_bytes(int N) {
  // s_s0 [128][32]; s_k, s_q [N][128]; s_x, s_y [N][N]; s_u, s_ks, s_qs
  // [N][32]; gamma, beta, alpha [N] (+1 pad); anc [N] (u64)
  return sizeof(float) * (static_cast<size_t>(kDk) * kCB + static_cast<size_t>(N) * kDk * 2 +
                          static_cast<size_t>(N) * N * 2 + static_cast<size_t>(N) * kCB * 3 +
                          3 * N + 1) +
         sizeof(uint64_t) * N + 16;
}

// 8 consecutive elements of an input row, loaded with 16-byte accesses
template <typename T>
struct Chunk8 {
  uint4 w[sizeof(T) / 2];
};

template <typename T>
__device__ __forceinline__ Chunk8<T> load8(const T* p) {
  Chunk8<T> c;
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(T) / 2); ++i) c.w[i] = reinterpret_cast<const uint4*>(p)[i];
  return c;
}

__device__ __forceinline__ void store8(float* dst, const Chunk8<uint16_t>& c) {
  const uint32_t w[4] = {c.w[0].x, c.w[0].y, c.w[0].z, c.w[0].w};
  float4 lo, hi;
  lo.x = __uint_as_float(w[0] << 16);
  lo.y = __uint_as_float(w[0] & 0xffff0000u);
  lo.z = __uint_as_float(w[1] << 16);
  lo.w = __uint_as_float(w[1] & 0xffff0000u);
  hi.x = __uint_as_float(w[2] << 16);
  hi.y = __uint_as_float(w[2] & 0xffff0000u);
  hi.z = __uint_as_float(w[3] << 16);
  hi.w = __uint_as_float(w[3] & 0xffff0000u);
  reinterpret_cast<float4*>(dst)[0] = lo;
  reinterpret_cast<float4*>(dst)[1] = hi;
}

__device__ __forceinline__ void store8(float* dst, const Chunk8<float>& c) {
  reinterpret_cast<uint4*>(dst)[0] = c.w[0];
  reinterpret_cast<uint4*>(dst)[1] = c.w[1];
}

template <typename T, typename TO>
__global__ __launch_bounds__(kThreads) void gdn_tree_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    const uint64_t* __restrict__ anc, int N, int H, int Dv, TO* __restrict__ out) {
  extern __shared__ __align__(16) float lds[];
  float* s_s0 = lds;                // [kDk][kCB]  this block's columns of S0
  float* s_k = s_s0 + kDk * kCB;    // [N][kDk]
  float* s_q = s_k + N * kDk;      // [N][kDk]
  float* s_x = s_q + N * kDk;      // [N][N]
  float* s_y = s_x + N * N;        // [N][N]
  float* s_u = s_y + N * N;        // [N][kCB]  V, then the right-hand side, then U
  float* s_ks = s_u + N * kCB;     // [N][kCB]  K S0
  float* s_qs = s_ks + N * kCB;    // [N][kCB]  Q S0
  float* s_gam = s_qs + N * kCB;   // [N]
  float* s_beta = s_gam + N;       // [N]
  float* s_alpha = s_beta + N;     // [N]
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(
      (reinterpret_cast<uintptr_t>(s_alpha + N) + 7) & ~static_cast<uintptr_t>(7));  // [N]
  __shared__ int s_maxdepth;

  const int ncb = Dv / kCB;
  const int cb = blockIdx.x % ncb;
  const int bh = blockIdx.x / ncb;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const uint64_t live = N >= 64 ? ~0ull : ((1ull << N) - 1ull);

  // ---- phase 0: tree, gates, keys and queries into LDS
  if (tid == 0) s_maxdepth = 1;
  for (int t = tid; t < N; t += kThreads) {
    const size_t nh = (static_cast<size_t>(b) * N + t) * H + h;
    s_alpha[t] = alpha[nh];
    s_beta[t] = beta[nh];
    // keep only real, earlier nodes (ancestors precede their descendants);
    // a node always sees itself
    const uint64_t below = t >= 63 ? ~0ull >> 1 : ((1ull << t) - 1ull);
    s_anc[t] = (anc[static_cast<size_t>(b) * N + t] & live & below) | (1ull << t);
  }
  {
    // keys and queries, 8 elements per chunk: every thread issues all of its
    // loads before converting any (N * 128 / 8 <= 1024 chunks, 4 per thread)
    constexpr int kPer = 4;
    const int nchunk = N * kDk / 8;
    Chunk8<T> ck[kPer], cq[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads;
      if (e < nchunk) {
        const int t = e / (kDk / 8), d = (e % (kDk / 8)) * 8;
        const size_t off = ((static_cast<size_t>(b) * N + t) * H + h) * kDk + d;
        ck[u] = load8(k + off);
        cq[u] = load8(q + off);
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = tid + u * kThreads;
      if (e < nchunk) {
        store8(s_k + e * 8, ck[u]);
        store8(s_q + e * 8, cq[u]);
      }
    }
  }
  {
    // the 128 x 32 column block of S0, as float4 (all loads in flight at once)
    const float* s0 = S0 + (static_cast<size_t>(b) * H + h) * kDk * Dv + cb * kCB;
    for (int e = tid; e < kDk * kCB / 4; e += kThreads) {
      const int d = e / (kCB / 4), c4 = e % (kCB / 4);
      reinterpret_cast<float4*>(s_s0)[e] =
          *reinterpret_cast<const float4*>(s0 + static_cast<size_t>(d) * Dv + 4 * c4);
    }
  }
  __syncthreads();

  // ---- phase 1: gamma, Gram terms, state products, V
  for (int t = tid; t < N; t += kThreads) {
    uint64_t m = s_anc[t];
    float gm = 1.0f;
    while (m) {
      const int i = __ffsll(static_cast<unsigned long long>(m)) - 1;
      gm *= s_alpha[i];
      m &= m - 1;
    }
    s_gam[t] = gm;
    atomicMax(&s_maxdepth, __popcll(s_anc[t]));
  }

  const int npairs = N * (N + 1) / 2;  // pairs (t, i) with i <= t
  for (int pidx = tid; pidx < npairs; pidx += kThreads) {
    int t = static_cast<int>((sqrtf(8.0f * pidx + 1.0f) - 1.0f) * 0.5f);
    while (t * (t + 1) / 2 > pidx) --t;
    while ((t + 1) * (t + 2) / 2 <= pidx) ++t;
    const int i = pidx - t * (t + 1) / 2;
    const uint64_t at = s_anc[t];
    float xv = 0.0f, yv = 0.0f;
    if ((at >> i) & 1ull) {
      uint64_t seg = at & ~s_anc[i];  // t's path strictly below i
      float r = 1.0f;
      while (seg) {
        const int s = __ffsll(static_cast<unsigned long long>(seg)) - 1;
        r *= s_alpha[s];
        seg &= seg - 1;
      }
      const float* kt = s_k + t * kDk;
      const float* ki = s_k + i * kDk;
      const float* qt = s_q + t * kDk;
      float kk = 0.0f, qk = 0.0f;
#pragma unroll 4
      for (int d = 0; d < kDk; d += 4) {
        const float4 a = *reinterpret_cast<const float4*>(kt + d);
        const float4 c = *reinterpret_cast<const float4*>(ki + d);
        const float4 e = *reinterpret_cast<const float4*>(qt + d);
        kk = fmaf(a.x, c.x, fmaf(a.y, c.y, fmaf(a.z, c.z, fmaf(a.w, c.w, kk))));
        qk = fmaf(e.x, c.x, fmaf(e.y, c.y, fmaf(e.z, c.z, fmaf(e.w, c.w, qk))));
      }
      yv = r * qk;
      if (i != t) xv = s_beta[t] * r * kk;
    }
    s_x[t * N + i] = xv;
    s_y[t * N + i] = yv;
  }

  {
    // K S0 and Q S0 for this column block: thread = (column c, node group),
    // four nodes per pass, four head dimensions per LDS read
    constexpr int kGroups = kThreads / kCB;
    const int c = tid % kCB;
    const int grp = tid / kCB;
    for (int t0 = grp; t0 < N; t0 += 4 * kGroups) {
      float ak[4] = {0.f, 0.f, 0.f, 0.f}, aq[4] = {0.f, 0.f, 0.f, 0.f};
      int tt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) tt[u] = min(t0 + u * kGroups, N - 1);
#pragma unroll 4
      for (int d = 0; d < kDk; d += 4) {
        const float s0a = s_s0[(d + 0) * kCB + c], s0b = s_s0[(d + 1) * kCB + c];
        const float s0c = s_s0[(d + 2) * kCB + c], s0d = s_s0[(d + 3) * kCB + c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 kv = *reinterpret_cast<const float4*>(s_k + tt[u] * kDk + d);
          const float4 qv = *reinterpret_cast<const float4*>(s_q + tt[u] * kDk + d);
          ak[u] = fmaf(kv.x, s0a, fmaf(kv.y, s0b, fmaf(kv.z, s0c, fmaf(kv.w, s0d, ak[u]))));
          aq[u] = fmaf(qv.x, s0a, fmaf(qv.y, s0b, fmaf(qv.z, s0c, fmaf(qv.w, s0d, aq[u]))));
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u * kGroups;
        if (t < N) {
          s_ks[t * kCB + c] = ak[u];
          s_qs[t * kCB + c] = aq[u];
          s_u[t * kCB + c] =
              load_f(v, ((static_cast<size_t>(b) * N + t) * H + h) * Dv + cb * kCB + c);
        }
      }
    }
  }
  __syncthreads();

  // ---- phase 2: right-hand side beta_t (v_t - gamma_t (K S0)_t)
  for (int e = tid; e < N * kCB; e += kThreads) {
    const int t = e / kCB;
    s_u[e] = s_beta[t] * (s_u[e] - s_gam[t] * s_ks[e]);
  }
  __syncthreads();

  // ---- phase 3: forward substitution, one depth level at a time
  const int maxdepth = s_maxdepth;
  for (int lvl = 2; lvl <= maxdepth; ++lvl) {
    for (int e = tid; e < N * kCB; e += kThreads) {
      const int t = e / kCB, c = e % kCB;
      const uint64_t at = s_anc[t];
      if (__popcll(at) != lvl) continue;
      uint64_t m = at & ~(1ull << t);
      float acc = s_u[e];
      while (m) {
        const int i = __ffsll(static_cast<unsigned long long>(m)) - 1;
        acc = fmaf(-s_x[t * N + i], s_u[i * kCB + c], acc);
        m &= m - 1;
      }
      s_u[e] = acc;
    }
    __syncthreads();
  }

  // ---- phase 4: outputs gamma_t (Q S0)_t + sum over ancestors-or-self of Y U
  for (int e = tid; e < N * kCB; e += kThreads) {
    const int t = e / kCB, c = e % kCB;
    uint64_t m = s_anc[t];
    float o = s_gam[t] * s_qs[e];
    while (m) {
      const int i = __ffsll(static_cast<unsigned long long>(m)) - 1;
      o = fmaf(s_y[t * N + i], s_u[i * kCB + c], o);
      m &= m - 1;
    }
    store_f(out, ((static_cast<size_t>(b) * N + t) * H + h) * Dv + cb * kCB + c, o);
  }
}

template <typename T, typename TO>
hipError_t launch_gdn_typed(const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                            int H, int Dv, void* out, hipStream_t stream) {
  const size_t lds = gdn_lds_bytes(N);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gdn_tree_kernel<T, TO>),
      hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(gdn_lds_bytes(64)));
  if (attr != hipSuccess) return attr;
  const unsigned grid = static_cast<unsigned>(B) * H * (Dv / kCB);
  hipLaunchKernelGGL((gdn_tree_kernel<T, TO>), dim3(grid), dim3(kThreads), lds, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     alpha, beta, S0, anc, N, H, Dv, static_cast<TO*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* S0, const uint64_t* anc, int B, int N, int H,
                      int Dk, int Dv, tv_dtype dtype, tv_dtype out_dtype, void* out,
                      hipStream_t stream) {
  (void)Dk;
  if (dtype == TV_BF16 && out_dtype == TV_BF16)
    return launch_gdn_typed<uint16_t, uint16_t>(q, k, v, alpha, beta, S0, anc, B, N, H, Dv, out,
                                                stream);
  if (dtype == TV_BF16 && out_dtype == TV_F32)
    return launch_gdn_typed<uint16_t, float>(q, k, v, alpha, beta, S0, anc, B, N, H, Dv, out,
                                             stream);
  if (dtype == TV_F32 && out_dtype == TV_F32)
    return launch_gdn_typed<float, float>(q, k, v, alpha, beta, S0, anc, B, N, H, Dv, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace tv
