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
// runs level by level over depth.
//
// Two kernels.  bf16 inputs: one workgroup per (sequence, head), with the
// dense products on MFMA (below).  fp32 inputs: workgroup = (sequence, head,
// 32 output columns), every product as fp32 FMAs from LDS; the columns of U
// and O are independent, so the state S0 is read once in total while the
// (small) Gram terms are recomputed per column block.
#include <atomic>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kDk = 128;
constexpr int kCB = 32;  // output columns per workgroup
constexpr int kThreads = 256;

__device__ __forceinline__ float load_f(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ void store_f(float* p, size_t i, float v) { p[i] = v; }

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

// Product of the gates over an ancestor set, exact at zero gates and free of
// underflow: the number of zero gates, and the product of the others as
// mant * 2^ex with |mant| in [0.5, 1).  Gates are multiplied in increasing node
// order, so a node's running product passes through its ancestors' products
// bit for bit and a ratio of two of them is the segment's product to within
// a few ulp.
struct GateProd {
  int zeros;
  int ex;
  float mant;
  __device__ float value() const { return zeros ? 0.0f : ldexpf(mant, ex); }
};

__device__ __forceinline__ GateProd gate_product(const float* alpha, uint64_t set) {
  GateProd g{0, 0, 1.0f};
  while (set) {
    const float a = alpha[__ffsll(static_cast<unsigned long long>(set)) - 1];
    set &= set - 1;
    if (a == 0.0f) {
      ++g.zeros;
    } else {
      int ea, em;
      g.mant *= frexpf(a, &ea);
      g.mant = frexpf(g.mant, &em);
      g.ex += ea + em;
    }
  }
  return g;
}

// gamma_t / gamma_i for i an ancestor of t (or t): the product of the gates
// strictly below i down to t; 0 when one of them is 0
__device__ __forceinline__ float gate_ratio(const int* zc, const float* mant, const float* rmant,
                                            const int* ex, int t, int i) {
  if (t == i) return 1.0f;
  if (zc[t] != zc[i]) return 0.0f;
  return ldexpf(mant[t] * rmant[i], ex[t] - ex[i]);
}

// ---------------------------------------------------------------------------
// bf16 inputs: the dense products on MFMA, one workgroup per (sequence, head).
//
// K S0 and Q S0 are one product [Q; K] S0, formed transposed (S0^T [Q; K]^T)
// so that S0's rows come out of LDS through the transpose read, as the value
// tile does in the attention kernel.  S0 is fp32; it is split into two bf16
// parts S0 = hi + lo (hi its round-to-nearest bf16, lo that of the remainder),
// so two bf16 products with fp32 accumulation carry S0 to ~16 mantissa bits
// while q and k are used exactly.  The Gram products [Q; K] K^T are exact bf16
// products; their masks and gate ratios are applied in registers.  The solve
// (I + X)^-1 is a short product of matrix powers on fp32 MFMA.  Gram products
// and solve need neither S0 nor v, so they run first, while S0's loads are in
// flight; the state products, the right-hand side and the outputs follow.
constexpr int kMThreads = 512;
constexpr int kRowB = kDk * 2;  // bytes of one bf16 row of 128

typedef __bf16 mbf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 mbf16x4_t __attribute__((ext_vector_type(4)));
typedef short ms16x4_t __attribute__((ext_vector_type(4)));
typedef short ms16x8_t __attribute__((ext_vector_type(8)));
typedef float mf32x4_t __attribute__((ext_vector_type(4)));

// 16-byte granules of a 256-byte bf16 row are XOR-swizzled by row, so reads
// of one granule column from 16 rows (and transpose reads of 4 rows) spread
// over the LDS banks
__device__ __forceinline__ int gswz(int row, int byte) {
  const int key = ((row & 7) << 1) | ((row >> 3) & 1);
  return row * kRowB + (((byte >> 4) ^ key) << 4) + (byte & 15);
}

__device__ __forceinline__ ms16x4_t tr_read(const unsigned char* p) {
  auto lp = (__attribute__((address_space(3))) mbf16x4_t*)(p);
  return __builtin_bit_cast(ms16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

constexpr int kUP = kDk + 16;  // row pitch of the right-hand side (floats): conflict-free column reads

// bytes of region 1: X, Y and two more NP x NP matrices for the solve, then one
// bf16 half of S0 at a time, then [Q; K] S0 (fp32, 2NP rows of 128)
__host__ __device__ inline size_t gdn_r1_bytes(int np) {
  const size_t half = static_cast<size_t>(kDk) * kRowB;
  const size_t qks = 2 * static_cast<size_t>(np) * kDk * 4;
  const size_t solve = 4 * static_cast<size_t>(np) * (np + 4) * 4;
  const size_t m = half > qks ? half : qks;
  return m > solve ? m : solve;
}

// bytes of the [Q; K] rows (bf16)
__host__ __device__ inline size_t gdn_r2_bytes(int np) { return 2 * static_cast<size_t>(np) * kRowB; }

size_t gdn_mfma_lds_bytes(int N) {
  const int np = (N + 15) / 16 * 16;
  // region 1; [Q; K]; V, later the right-hand side (fp32); M (fp32); alpha,
  // beta, gamma, the gate-product mantissa and its reciprocal, depth, zero
  // count, exponent, ancestor words.  Up to 32 nodes this is 73 KB, so two
  // workgroups fit a CU.
  return gdn_r1_bytes(np) + gdn_r2_bytes(np) + static_cast<size_t>(np) * kUP * 4 +
         static_cast<size_t>(np) * (np + 4) * 4 + 64 * 4 * 8 + 64 * 8;
}

// One 16 x 16 tile (row tile rt, column tile ct) of C = A B (+ D), NP x NP
// fp32 matrices of row pitch mp in LDS, on v_mfma_f32_16x16x4f32; B's
// entries are scaled by `sb`.  A lane holds column lr of rows 4 lg .. 4 lg + 3.
template <bool kAdd, int kNT>
__device__ __forceinline__ void gdn_mm_tile(const float* A, const float* B, const float* Dm, float* C, int mp,
                                            int rt, int ct, int lr, int lg, float sb) {
  mf32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kAdd) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = Dm[(16 * rt + 4 * lg + r) * mp + 16 * ct + lr];
  }
#pragma unroll
  for (int ks = 0; ks < 4 * kNT; ++ks) {
    const float a = A[(16 * rt + lr) * mp + 4 * ks + lg];
    const float bv = sb * B[(4 * ks + lg) * mp + 16 * ct + lr];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(16 * rt + 4 * lg + r) * mp + 16 * ct + lr] = acc[r];
}

// One step of the solve as a single phase: Mo = M + M (sb P) and, when Po is
// given, Po = P P.  Both read only M and P, so their 2 kNT^2 tiles are dealt
// to the 8 waves together.  kNT = NP / 16 tiles per side.
template <int kNT>
__device__ __forceinline__ void gdn_solve_step(const float* M, const float* P, float* Mo, float* Po, int mp,
                                               int wave, int lr, int lg, float sb) {
  constexpr int kT = kNT * kNT;
#pragma unroll
  for (int mm = 0; mm < (2 * kT + 7) / 8; ++mm) {
    const int u = wave + 8 * mm;
    if (u < kT) {
      gdn_mm_tile<true, kNT>(M, P, M, Mo, mp, u / kNT, u % kNT, lr, lg, sb);
    } else if (u < 2 * kT && Po != nullptr) {
      const int v = u - kT;
      gdn_mm_tile<false, kNT>(P, P, nullptr, Po, mp, v / kNT, v % kNT, lr, lg, 1.0f);
    }
  }
}

// kM: node tiles of 16 rows in [Q; K], 2 NP / 16 for NP = N rounded up to 16.
// Up to 32 nodes (kM <= 4) the kernel fits two workgroups per CU, registers
// included.
template <typename TO, int kM>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(kM <= 4 ? 4 : 2))) void gdn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    const uint64_t* __restrict__ anc, int N, int H, TO* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NP = 8 * kM;  // N rounded up to 16 (the launch picks kM)
  constexpr int MP = NP + 4;                     // row pitch of the NP x NP matrices (floats)
  unsigned char* r1 = smem;                      // X, Y, third; then S0 hi, S0 lo; then [Q; K] S0 fp32
  unsigned char* r2 = smem + gdn_r1_bytes(NP);   // [Q; K] bf16 [2NP][128]
  float* s_u = reinterpret_cast<float*>(r2 + gdn_r2_bytes(NP));  // V, then the right-hand side
  float* s_m = s_u + NP * kUP;                   // M [NP][MP]
  float* s_alpha = s_m + NP * MP;
  float* s_beta = s_alpha + 64;
  float* s_gam = s_beta + 64;
  float* s_mant = s_gam + 64;   // gate product over nonzero gates: mantissa,
  float* s_rmant = s_mant + 64; // its reciprocal,
  int* s_depth = reinterpret_cast<int*>(s_rmant + 64);
  int* s_zc = s_depth + 64;     // zero gates on the root path,
  int* s_ex = s_zc + 64;        // and the binary exponent of the product
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(s_ex + 64);
  __shared__ int s_maxdepth;

  const int bh = blockIdx.x;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const uint64_t live = N >= 64 ? ~0ull : ((1ull << N) - 1ull);

  // ---- phase 0: q and k rows, v and the gates, then S0.  S0's loads stay in
  // flight through the Gram products and the solve, which do not need it.
  if (tid == 0) s_maxdepth = 1;
  constexpr int kQKPer = 2 * 64 * (kRowB / 16) / kMThreads;  // q / k granules per thread (at most)
  constexpr int kVPer = 64 * (kDk / 8) / kMThreads;           // v granules per thread (at most)
  uint4 gq[kQKPer], gv[kVPer];
#pragma unroll
  for (int u = 0; u < kQKPer; ++u) {
    const int e = tid + u * kMThreads;
    const int row = e / (kRowB / 16), gr = e % (kRowB / 16);
    const bool isk = row >= NP;
    const int t = isk ? row - NP : row;
    gq[u] = make_uint4(0, 0, 0, 0);
    if (row < 2 * NP && t < N)
      gq[u] = *reinterpret_cast<const uint4*>((isk ? k : q) +
                                              ((static_cast<size_t>(b) * N + t) * H + h) * kDk + gr * 8);
  }
#pragma unroll
  for (int u = 0; u < kVPer; ++u) {
    const int e = tid + u * kMThreads;
    const int t = e / (kDk / 8), gr = e % (kDk / 8);
    gv[u] = make_uint4(0, 0, 0, 0);
    if (t < N)
      gv[u] = *reinterpret_cast<const uint4*>(v + ((static_cast<size_t>(b) * N + t) * H + h) * kDk +
                                              gr * 8);
  }
  float ga = 1.0f, gb = 0.0f;
  uint64_t gw = 0ull;
  if (tid < N) {
    const size_t nh = (static_cast<size_t>(b) * N + tid) * H + h;
    ga = alpha[nh];
    gb = beta[nh];
    gw = anc[static_cast<size_t>(b) * N + tid];
  }
#pragma unroll
  for (int u = 0; u < kQKPer; ++u) {
    const int e = tid + u * kMThreads;
    const int row = e / (kRowB / 16), gr = e % (kRowB / 16);
    if (row < 2 * NP) *reinterpret_cast<uint4*>(r2 + gswz(row, gr * 16)) = gq[u];
  }
#pragma unroll
  for (int u = 0; u < kVPer; ++u) {
    const int e = tid + u * kMThreads;
    const int t = e / (kDk / 8), gr = e % (kDk / 8);
    if (t < NP) {  // rows past N are zero (they meet zero weights in the products)
      const uint4 w = gv[u];
      float4 lo, hi;
      lo.x = __uint_as_float(w.x << 16); lo.y = __uint_as_float(w.x & 0xffff0000u);
      lo.z = __uint_as_float(w.y << 16); lo.w = __uint_as_float(w.y & 0xffff0000u);
      hi.x = __uint_as_float(w.z << 16); hi.y = __uint_as_float(w.z & 0xffff0000u);
      hi.z = __uint_as_float(w.w << 16); hi.w = __uint_as_float(w.w & 0xffff0000u);
      reinterpret_cast<float4*>(s_u + t * kUP + gr * 8)[0] = lo;
      reinterpret_cast<float4*>(s_u + t * kUP + gr * 8)[1] = hi;
    }
  }
  if (tid < 64) {
    const int t = tid;
    s_alpha[t] = ga;
    s_beta[t] = gb;
    // keep only real, earlier nodes (ancestors precede their descendants);
    // a node always sees itself
    const uint64_t below = t >= 63 ? ~0ull >> 1 : ((1ull << t) - 1ull);
    s_anc[t] = t < N ? ((gw & live & below) | (1ull << t)) : 0ull;
  }
  __syncthreads();
  // S0 goes out once the small loads are in (issued with them, it would
  // delay them: every workgroup's S0 competes for HBM at the same moment),
  // in three batches between the phases that do not need it, so that no
  // wave stalls long on a full memory pipeline
  const float* s0 = S0 + static_cast<size_t>(bh) * kDk * kDk;
  float4 f[8];
  auto s0_issue = [&](int u0, int u1) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u >= u0 && u < u1) f[u] = reinterpret_cast<const float4*>(s0)[tid + u * kMThreads];
  };
  s0_issue(0, 3);
  if (tid < 64) {
    // gamma_t = product of alpha over t's root path, kept as a count of zero
    // gates and the product of the others as mantissa * 2^exponent
    const int t = tid;
    const GateProd gp = gate_product(s_alpha, s_anc[t]);
    s_gam[t] = gp.value();
    s_mant[t] = gp.mant;
    s_rmant[t] = 1.0f / gp.mant;
    s_zc[t] = gp.zeros;
    s_ex[t] = gp.ex;
    const int dpt = __popcll(s_anc[t]);
    s_depth[t] = dpt;
    if (t < N) atomicMax(&s_maxdepth, dpt);
  }

  // ---- phase 1: the Gram products [Q; K] K^T on MFMA (exact bf16 products)
  constexpr int nqks = NP;              // 8 column tiles x 2NP / 16 node tiles
  constexpr int ngram = NP * NP / 128;  // 2NP / 16 row tiles x NP / 16 key tiles
  mf32x4_t qks[kM], gram[kM / 2];
#pragma unroll
  for (int m = 0; m < kM / 2; ++m) {
    const int u = wave + 8 * m;
    gram[m] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
    if (u < ngram) {
      const int kt = u % (NP / 16), rt = u / (NP / 16);
#pragma unroll
      for (int ks = 0; ks < kDk / 32; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(r2 + gswz(16 * rt + lr, 2 * (32 * ks + 8 * lg)));
        const uint4 bk = *reinterpret_cast<const uint4*>(r2 + gswz(NP + 16 * kt + lr, 2 * (32 * ks + 8 * lg)));
        gram[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8_t, a),
                                                           __builtin_bit_cast(mbf16x8_t, bk), gram[m],
                                                           0, 0, 0);
      }
    }
  }
  s0_issue(3, 6);
  __syncthreads();  // gamma and the depths are in

  // X and Y with their masks and gate ratios, into region 1
  float* s_x = reinterpret_cast<float*>(r1);  // [NP][MP]
  float* s_y = s_x + NP * MP;                 // [NP][MP]
  float* s_t = s_y + NP * MP;                 // [NP][MP], two more matrices for the solve
  float* s_t2 = s_t + NP * MP;                // [NP][MP]
#pragma unroll
  for (int m = 0; m < kM / 2; ++m) {
    const int u = wave + 8 * m;
    if (u < ngram) {
      const int kt = u % (NP / 16), rt = u / (NP / 16);
      const int i = 16 * kt + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * lg + r;
        if (row < NP) {
          // a query row: Y over ancestors-or-self
          const int t = row;
          float y = 0.0f;
          if (t < N && i < N && ((s_anc[t] >> i) & 1ull))
            y = gate_ratio(s_zc, s_mant, s_rmant, s_ex, t, i) * gram[m][r];
          s_y[t * MP + i] = y;
        } else {
          // a key row: X over strict ancestors
          const int t = row - NP;
          float x = 0.0f;
          if (t < N && i < N && i != t && ((s_anc[t] >> i) & 1ull))
            x = s_beta[t] * gate_ratio(s_zc, s_mant, s_rmant, s_ex, t, i) * gram[m][r];
          s_x[t * MP + i] = x;
        }
      }
    }
  }
  __syncthreads();

  s0_issue(6, 8);

  // ---- phase 2: M = Y (I + X)^-1.  X only couples a node to its strict
  // ancestors, so X^d = 0 past the tree's depth and (I + X)^-1 is the finite
  // product of (I + (-X)^(2^j)), j < ceil(log2 depth): M starts as Y and takes
  // one factor per step, while the power is squared for the next step (both
  // products in one phase, one barrier per step).  Four NP x NP buffers
  // rotate; fp32 MFMA throughout.
  {
    const int maxdepth = s_maxdepth;
    int steps = 0;
    while ((1 << steps) < maxdepth) ++steps;
    float* bm = s_y;   // M
    float* bp = s_x;   // the power of X, stored as X^(2^j) ((-X)^(2^j) for j > 0 is the same)
    float* fm = s_t;   // free, for the next M
    float* fp = s_t2;  // free, for the next power
    constexpr int nt = NP / 16;
    for (int j = 0; j < steps; ++j) {
      const bool more = j + 1 < steps;
      // M <- M + M (-X)^(2^j): the power is X negated for j = 0, else as stored
      gdn_solve_step<nt>(bm, bp, fm, more ? fp : nullptr, MP, wave, lr, lg, j == 0 ? -1.0f : 1.0f);
      __syncthreads();
      float* tmp = bm;
      bm = fm;
      fm = tmp;
      if (more) {
        tmp = bp;
        bp = fp;
        fp = tmp;
      }
    }
    // M out of region 1, which S0 takes next
    for (int e = tid; e < NP * MP / 4; e += kMThreads)
      reinterpret_cast<float4*>(s_m)[e] = reinterpret_cast<const float4*>(bm)[e];
  }
  __syncthreads();

  // ---- phase 3: [Q; K] S0 on MFMA, formed transposed (S0^T [Q; K]^T).  S0
  // is split into bf16 hi = bf16(S0) (round to nearest even, the hardware
  // conversion) and lo = bf16(S0 - hi); the halves pass one after the other
  // through region 1, lo waiting packed in registers.
  uint2 s0lo[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid + u * kMThreads;
    const int d = e >> 5, c = (e & 31) * 4;
    const mbf16x4_t hv = {static_cast<__bf16>(f[u].x), static_cast<__bf16>(f[u].y),
                          static_cast<__bf16>(f[u].z), static_cast<__bf16>(f[u].w)};
    const mbf16x4_t lv = {static_cast<__bf16>(f[u].x - static_cast<float>(hv[0])),
                          static_cast<__bf16>(f[u].y - static_cast<float>(hv[1])),
                          static_cast<__bf16>(f[u].z - static_cast<float>(hv[2])),
                          static_cast<__bf16>(f[u].w - static_cast<float>(hv[3]))};
    *reinterpret_cast<uint2*>(r1 + gswz(d, 2 * c)) = __builtin_bit_cast(uint2, hv);
    s0lo[u] = __builtin_bit_cast(uint2, lv);
  }
  __syncthreads();
  // Tile u = wave + 8 m is column tile `wave` of node tile m: a wave keeps one
  // column tile, so each k-step reads its S0 fragment once for all node tiles.
  auto s0_product = [&]() {
    const int vcol = wave * 32 + 8 * (lr & 3);
#pragma unroll
    for (int ks = 0; ks < kDk / 32; ++ks) {
      const int vrow = 32 * ks + 4 * lg + (lr >> 2);
      const ms16x4_t h0 = tr_read(r1 + gswz(vrow, vcol));
      const ms16x4_t h1 = tr_read(r1 + gswz(vrow + 16, vcol));
      const ms16x8_t ah = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        if (wave + 8 * m < nqks) {
          const int row = 16 * m + lr;
          const uint2 b0 = *reinterpret_cast<const uint2*>(r2 + gswz(row, 2 * (32 * ks + 4 * lg)));
          const uint2 b1 = *reinterpret_cast<const uint2*>(r2 + gswz(row, 2 * (32 * ks + 16 + 4 * lg)));
          const mbf16x8_t bb = __builtin_bit_cast(mbf16x8_t, make_uint4(b0.x, b0.y, b1.x, b1.y));
          qks[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8_t, ah), bb,
                                                            qks[m], 0, 0, 0);
        }
      }
    }
  };
#pragma unroll
  for (int m = 0; m < kM; ++m) qks[m] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
  s0_product();  // high half
  __syncthreads();  // every read of S0's high half is done
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = tid + u * kMThreads;
    const int d = e >> 5, c = (e & 31) * 4;
    *reinterpret_cast<uint2*>(r1 + gswz(d, 2 * c)) = s0lo[u];
  }
  __syncthreads();
  s0_product();  // low half
  __syncthreads();  // every read of S0 is done

  // [Q; K] S0 rows into region 1
  float* s_qks = reinterpret_cast<float*>(r1);  // [2NP][128]
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int u = wave + 8 * m;
    if (u < nqks) {
      const int ct = u & 7, nt = u >> 3;
      *reinterpret_cast<float4*>(s_qks + (16 * nt + lr) * kDk + 16 * ct + 4 * lg) =
          make_float4(qks[m][0], qks[m][1], qks[m][2], qks[m][3]);
    }
  }
  __syncthreads();

  // ---- phase 4: right-hand side beta_t (v_t - gamma_t (K S0)_t), in place of V
  for (int e = tid; e < N * (kDk / 4); e += kMThreads) {
    const int t = e / (kDk / 4), c = (e % (kDk / 4)) * 4;
    float4 uu = *reinterpret_cast<const float4*>(s_u + t * kUP + c);
    const float4 ks = *reinterpret_cast<const float4*>(s_qks + (NP + t) * kDk + c);
    const float bt = s_beta[t], gt = s_gam[t];
    uu.x = bt * (uu.x - gt * ks.x);
    uu.y = bt * (uu.y - gt * ks.y);
    uu.z = bt * (uu.z - gt * ks.z);
    uu.w = bt * (uu.w - gt * ks.w);
    *reinterpret_cast<float4*>(s_u + t * kUP + c) = uu;
  }
  __syncthreads();

  // ---- phase 5: O^T = (right-hand side)^T M^T + gamma (Q S0)^T, tiles of
  // 16 state columns x 16 nodes; a lane ends with 4 consecutive columns of
  // one node's output
  constexpr int nt = NP / 16;
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int u = wave + 8 * mm;
    if (u < 8 * nt) {
      const int ct = u & 7, ntile = u >> 3;
      const int t = 16 * ntile + lr;
      const float gt = s_gam[t];
      const float4 qs = *reinterpret_cast<const float4*>(s_qks + t * kDk + 16 * ct + 4 * lg);
      mf32x4_t acc = {gt * qs.x, gt * qs.y, gt * qs.z, gt * qs.w};
#pragma unroll
      for (int ks = 0; ks < NP / 4; ++ks) {
        const float a = s_u[(4 * ks + lg) * kUP + 16 * ct + lr];
        const float bv = s_m[t * MP + 4 * ks + lg];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
      }
      if (t < N) {
        const size_t off = ((static_cast<size_t>(b) * N + t) * H + h) * kDk + 16 * ct + 4 * lg;
        if constexpr (sizeof(TO) == 2) {
          const mbf16x4_t w = {static_cast<__bf16>(acc[0]), static_cast<__bf16>(acc[1]),
                               static_cast<__bf16>(acc[2]), static_cast<__bf16>(acc[3])};
          *reinterpret_cast<uint2*>(out + off) = __builtin_bit_cast(uint2, w);
        } else {
          *reinterpret_cast<float4*>(out + off) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
  }
}

// Raises a kernel's dynamic LDS limit once per device (the attribute is held
// per device); `done` holds one flag per device id.
constexpr int kMaxDevices = 64;
hipError_t max_lds_once(std::atomic<int>* done, const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && cached) done[dev].store(1, std::memory_order_release);
  return e;
}

// A grid that fits the CUs one workgroup each asks for more LDS than half a
// CU's, so that no two of its workgroups share a CU.
constexpr size_t kGdnSpreadLds = 81 * 1024;

template <typename TO, int kM>
hipError_t launch_gdn_mfma_m(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                             int H, void* out, hipStream_t stream) {
  const size_t most = gdn_mfma_lds_bytes(8 * kM);
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t attr = max_lds_once(lds_set, reinterpret_cast<const void*>(&gdn_mfma_kernel<TO, kM>),
                                       static_cast<int>(most > kGdnSpreadLds ? most : kGdnSpreadLds));
  if (attr != hipSuccess) return attr;
  size_t lds = gdn_mfma_lds_bytes(N);
  if (static_cast<long long>(B) * H <= device_cus() && lds < kGdnSpreadLds) lds = kGdnSpreadLds;
  hipLaunchKernelGGL((gdn_mfma_kernel<TO, kM>), dim3(static_cast<unsigned>(B) * H), dim3(kMThreads),
                     lds, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), alpha, beta, S0,
                     anc, N, H, static_cast<TO*>(out));
  return hipGetLastError();
}

template <typename TO>
hipError_t launch_gdn_mfma(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                           int H, void* out, hipStream_t stream) {
  switch ((N + 15) / 16) {
    case 1: return launch_gdn_mfma_m<TO, 2>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    case 2: return launch_gdn_mfma_m<TO, 4>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    case 3: return launch_gdn_mfma_m<TO, 6>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    case 4: return launch_gdn_mfma_m<TO, 8>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename TO>
hipError_t launch_gdn_typed(const void* q, const void* k, const void* v, const float* alpha,
                            const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                            int H, int Dv, void* out, hipStream_t stream) {
  const size_t lds = gdn_lds_bytes(N);
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t attr = max_lds_once(lds_set, reinterpret_cast<const void*>(&gdn_tree_kernel<T, TO>),
                                       static_cast<int>(gdn_lds_bytes(64)));
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
    return launch_gdn_mfma<uint16_t>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
  if (dtype == TV_BF16 && out_dtype == TV_F32)
    return launch_gdn_mfma<float>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
  if (dtype == TV_F32 && out_dtype == TV_F32)
    return launch_gdn_typed<float, float>(q, k, v, alpha, beta, S0, anc, B, N, H, Dv, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace tv
