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
// same system.  The columns of U and O are independent, so a kernel may split
// the state's columns over workgroups: S0 is still read once in total, while
// the small node-by-node terms are formed again per column block.
//
// Three kernels.  bf16 inputs up to 32 nodes: one 8-wave workgroup per
// (sequence, head), the dense products on MFMA and the solve as a product of
// matrix powers.  bf16 inputs past 32 nodes: one 8-wave workgroup per
// (sequence, head) too, only the tiles on or below the block diagonal, and a
// block-row solve on MFMA.  fp32 inputs: every product as fp32 FMAs, the
// solve level by level over depth.
#include <atomic>

#include "tv_internal.h"

// bf16 trees of at least this many nodes take the block-triangular kernel
// (gdn_tri_kernel); smaller ones the dense one (gdn_head_kernel), which fits
// two workgroups per CU up to 32 nodes.  Measured warm at H = 16: from 33
// nodes on the block-triangular kernel is faster at B = 16 and B = 32 (at 56
// nodes 13.9 against 20.0 us and 26.4 against 39.6 us); at 32 nodes and B = 32
// the dense kernel is (15.0 against 20.9 us).
#ifndef TV_GDN_TRI_FROM
#define TV_GDN_TRI_FROM 33
#endif

namespace tv {

namespace {

constexpr int kDk = 128;         // Dk = Dv
constexpr int kGC = 32;          // state columns per workgroup of the fp32 kernel
constexpr int kNCB = kDk / kGC;  // column blocks per (sequence, head)
constexpr int kGThreads = 256;

// Workgroup -> (sequence-head bh, column block cb) for ncb column blocks per
// (sequence, head).  Workgroups are dealt to the 8 XCDs round-robin by index,
// so the column blocks of one (sequence, head) get indices equal mod 8: they
// share an XCD and its L2, and their q and k rows come from HBM once.
// Returns false for the padding workgroups of a grid rounded up to 8
// (sequence, head) pairs.
__device__ __forceinline__ bool gdn_block(int wgi, int BH, int ncb, int* bh, int* cb) {
  const int xcd = wgi & 7, slot = wgi >> 3;
  *cb = slot % ncb;
  *bh = (slot / ncb) * 8 + xcd;
  return *bh < BH;
}

unsigned gdn_grid(int BH, int ncb) { return static_cast<unsigned>((BH + 7) / 8) * 8u * ncb; }

// Ancestor word `word` of node t, restricted to real, earlier nodes
// (ancestors precede their descendants) plus t itself.
__device__ __forceinline__ uint64_t anc_clean(uint64_t w, int t, int word) {
  const int lo = 64 * word;
  uint64_t below;
  if (t >= lo + 64) below = ~0ull;
  else if (t <= lo) below = 0ull;
  else below = (1ull << (t - lo)) - 1ull;
  const uint64_t self = (t >= lo && t < lo + 64) ? (1ull << (t - lo)) : 0ull;
  return (w & below) | self;
}

typedef __bf16 gbf16x8_t __attribute__((ext_vector_type(8)));
typedef float gf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowB = kDk * 2;  // bytes of one bf16 row of 128

// 16-byte granules of a 256-byte bf16 row are XOR-swizzled by row, so reads
// of one granule column from 16 rows spread over the LDS banks
__device__ __forceinline__ int gswz(int row, int byte) {
  const int key = ((row & 7) << 1) | ((row >> 3) & 1);
  return row * kRowB + (((byte >> 4) ^ key) << 4) + (byte & 15);
}

// ---------------------------------------------------------------------------
// bf16 inputs, N < TV_GDN_TRI_FROM (up to 64 supported): the dense products on
// MFMA, one 8-wave workgroup per (sequence, head).
//
// K S0 and Q S0 are one product [Q; K] S0 whose S0 operand never passes
// through LDS: each wave owns 16 state columns, loads them from HBM in 16-byte
// pieces, and a 4 x 4 transpose inside each quad of lanes leaves every lane
// the eight rows of one column that the matrix-core operand layout gives it.
// S0 is fp32; it is split into two bf16 parts S0 = hi + lo (hi its
// round-to-nearest bf16, lo that of the remainder), so two bf16 products with
// fp32 accumulation carry S0 to ~16 mantissa bits while q and k are used
// exactly.  The Q rows are formed transposed (S0^T Q^T), which leaves each lane
// one node's outputs for four consecutive columns, the layout the output
// product accumulates in; the K rows are formed as K S0 with the node rows
// permuted so that each lane holds, for one column, the nodes the output
// product takes as its contraction operand.  The right-hand side is then made
// in registers and no barrier follows the state products.  The Gram products
// [Q; K] K^T are exact bf16 products; their masks and gate ratios are applied
// in registers.  The solve (I + X)^-1 is a short product of matrix powers on
// fp32 MFMA.  Gram products and solve need neither S0 nor v, so they run
// first, while S0's loads are in flight.
constexpr int kMThreads = 512;

typedef __bf16 mbf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 mbf16x4_t __attribute__((ext_vector_type(4)));
typedef float mf32x4_t __attribute__((ext_vector_type(4)));

// one quad_perm lane exchange (DPP): lane i of each quad of lanes takes the
// value of lane perm[i]
template <int kCtrl>
__device__ __forceinline__ float quad_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}

// 4 x 4 transpose inside each quad of lanes: lane b of a quad holds row b of
// a block and returns column b, in two exchanges, first with lane b ^ 1 (the
// odd or even columns), then with lane b ^ 2 (the column pairs)
__device__ __forceinline__ float4 quad_transpose(float4 x, int b) {
  const bool odd = b & 1, hi = b & 2;
  const float a0 = quad_dpp<0xb1>(odd ? x.x : x.y), a1 = quad_dpp<0xb1>(odd ? x.z : x.w);
  const float y0 = odd ? a0 : x.x, y1 = odd ? x.y : a0, y2 = odd ? a1 : x.z, y3 = odd ? x.w : a1;
  const float c0 = quad_dpp<0x4e>(hi ? y0 : y2), c1 = quad_dpp<0x4e>(hi ? y1 : y3);
  return hi ? make_float4(c0, c1, y2, y3) : make_float4(y0, y1, c0, c1);
}

constexpr int kHUP = kDk + 16;  // row pitch of the right-hand side (floats): conflict-free column reads

// bytes of region 1: X, Y and two more NP x NP matrices for the solve; M is
// left in one of them
__host__ __device__ inline size_t gdn_r1_bytes(int np) { return 4 * static_cast<size_t>(np) * (np + 4) * 4; }

// bytes of the [Q; K] rows (bf16)
__host__ __device__ inline size_t gdn_r2_bytes(int np) { return 2 * static_cast<size_t>(np) * kRowB; }

size_t gdn_mfma_lds_bytes(int N) {
  const int np = (N + 15) / 16 * 16;
  // region 1; [Q; K]; V (fp32); beta, gamma, the gate-product mantissa and its
  // reciprocal, zero count, exponent, ancestor words.  Up to 32 nodes this is
  // 54 KB, so two workgroups fit a CU.
  return gdn_r1_bytes(np) + gdn_r2_bytes(np) + static_cast<size_t>(np) * kHUP * 4 + 64 * 4 * 6 + 64 * 8;
}

// One 16 x 16 tile (row tile rt, column tile ct) of C = A B (+ D), NP x NP
// fp32 matrices of row pitch mp in LDS, on v_mfma_f32_16x16x4f32; B's
// entries are scaled by `sb`.  A lane holds column lr of rows 4 lg .. 4 lg + 3.
// A and B are lower triangular (a node couples only to itself and its
// ancestors, which precede it): only k-tiles ct .. rt contribute, and a tile
// above the diagonal is zero.  Two accumulators halve the dependent chain.
template <bool kAdd, int kNT>
__device__ __forceinline__ void gdn_mm_tile(const float* A, const float* B, const float* Dm, float* C, int mp,
                                            int rt, int ct, int lr, int lg, float sb) {
  mf32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kAdd) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = Dm[(16 * rt + 4 * lg + r) * mp + 16 * ct + lr];
  }
#pragma unroll
  for (int ks = 0; ks < 4 * kNT; ks += 2) {
    if (ks >= 4 * ct && ks < 4 * rt + 4) {
      const float a = A[(16 * rt + lr) * mp + 4 * ks + lg];
      const float bv = sb * B[(4 * ks + lg) * mp + 16 * ct + lr];
      const float a2 = A[(16 * rt + lr) * mp + 4 * ks + 4 + lg];
      const float bv2 = sb * B[(4 * ks + 4 + lg) * mp + 16 * ct + lr];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, bv2, acc2, 0, 0, 0);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(16 * rt + 4 * lg + r) * mp + 16 * ct + lr] = acc[r] + acc2[r];
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
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(kM <= 4 ? 4 : 2))) void gdn_head_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    const uint64_t* __restrict__ anc, int N, int H, TO* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NP = 8 * kM;  // N rounded up to 16 (the launch picks kM)
  constexpr int MP = NP + 4;                     // row pitch of the NP x NP matrices (floats)
  unsigned char* r1 = smem;                      // X, Y and two more NP x NP matrices for the solve
  unsigned char* r2 = smem + gdn_r1_bytes(NP);   // [Q; K] bf16 [2NP][128]
  float* s_u = reinterpret_cast<float*>(r2 + gdn_r2_bytes(NP));  // V [NP][kHUP]
  float* s_beta = s_u + NP * kHUP;
  float* s_gam = s_beta + 64;
  float* s_mant = s_gam + 64;   // gate product over nonzero gates: mantissa,
  float* s_rmant = s_mant + 64; // its reciprocal,
  int* s_zc = reinterpret_cast<int*>(s_rmant + 64);  // zero gates on the root path,
  int* s_ex = s_zc + 64;        // and the binary exponent of the product
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(s_ex + 64);
  __shared__ int s_steps;       // ceil(log2(depth of the deepest node))

  const int bh = blockIdx.x;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const uint64_t live = N >= 64 ? ~0ull : ((1ull << N) - 1ull);

  // ---- phase 0: q and k rows, v and the gates, then S0.  S0's loads stay in
  // flight through the Gram products and the solve, which do not need it.
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
  // S0 goes out in three batches: the first right after the small loads
  // are issued (behind them in the memory pipeline, so it does not hold them
  // back), the others between the phases that do not need it, so that no
  // wave stalls long on a full memory pipeline (issued all at once, or ahead
  // of the gates and ancestor words, S0 delayed the small loads and the
  // kernel took longer).  Wave w owns state columns 16w .. 16w + 15.  Load
  // u = 2 ks + hf gives lane (lr, lg) = (4 q + b, lg) the four columns
  // 16 w + 4 q .. + 3 of row 32 ks + 8 lg + 4 hf + b (16 rows of 64 bytes per
  // instruction; 16-byte loads keep the instruction count low, which matters
  // while misses are slow); a 4 x 4 transpose inside each quad of lanes then
  // leaves lane (lr, lg) rows 32 ks + 8 lg + j, j < 8, of column 16 w + lr:
  // the bf16 operand layout of the state products.
  const float* s0 = S0 + static_cast<size_t>(bh) * kDk * kDk + 16 * wave + 4 * (lr >> 2);
  float4 f[kDk / 16];
  auto s0_issue = [&](int u0, int u1) {
#pragma unroll
    for (int u = 0; u < kDk / 16; ++u)
      if (u >= u0 && u < u1)
        f[u] = *reinterpret_cast<const float4*>(s0 + (32 * (u >> 1) + 8 * lg + 4 * (u & 1) + (lr & 3)) * kDk);
  };
  s0_issue(0, 3);
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
      reinterpret_cast<float4*>(s_u + t * kHUP + gr * 8)[0] = lo;
      reinterpret_cast<float4*>(s_u + t * kHUP + gr * 8)[1] = hi;
    }
  }
  if (tid < 64) {
    // Wave 0, lane t = node t: gamma_t, the product of alpha over t's root
    // path, kept as a count of zero gates and the product of the others as
    // mant * 2^ex (|mant| in [0.5, 1)), by pointer jumping: (mant, ex, zeros)
    // covers the path segment (jmp, t], and a round appends the segment that
    // ends at jmp, doubling the reach.  Rounds run until every node has
    // reached its root: ceil(log2(depth)) of them, the step count of the solve.
    const int t = tid;
    s_beta[t] = gb;
    // keep only real, earlier nodes (ancestors precede their descendants);
    // a node always sees itself
    const uint64_t below = t >= 63 ? ~0ull >> 1 : ((1ull << t) - 1ull);
    const uint64_t strict = t < N ? (gw & live & below) : 0ull;
    s_anc[t] = t < N ? (strict | (1ull << t)) : 0ull;
    int jmp = strict ? 63 - __clzll(static_cast<long long>(strict)) : -1;
    int zeros = (t < N && ga == 0.0f) ? 1 : 0;
    int ex = 1;
    float mant = 0.5f;
    if (!zeros) mant = frexpf(ga, &ex);
    int rounds = 0;
    while (__ballot(jmp >= 0)) {
      const int src = jmp >= 0 ? jmp : t;
      const float mj = __shfl(mant, src, 64);
      const int ej = __shfl(ex, src, 64), zj = __shfl(zeros, src, 64), pj = __shfl(jmp, src, 64);
      if (jmp >= 0) {
        int e2;
        mant = frexpf(mant * mj, &e2);
        ex += ej + e2;
        zeros += zj;
        jmp = pj;
      }
      ++rounds;
    }
    s_gam[t] = zeros ? 0.0f : ldexpf(mant, ex);
    s_mant[t] = mant;
    s_rmant[t] = 1.0f / mant;
    s_zc[t] = zeros;
    s_ex[t] = ex;
    if (t == 0) s_steps = rounds;
  }
  __syncthreads();

  // ---- phase 1: the Gram products [Q; K] K^T on MFMA (exact bf16 products)
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

  // X and Y with their masks and gate ratios, into region 1
  float* s_x = reinterpret_cast<float*>(r1);  // [NP][MP]
  float* s_y = s_x + NP * MP;                 // [NP][MP]
  float* s_t = s_y + NP * MP;                 // [NP][MP], two more matrices for the solve
  float* s_t2 = s_t + NP * MP;                // [NP][MP]
  // Query rows give Y over ancestors-or-self, key rows X over strict
  // ancestors (times beta_t).  Every operand is read before any is used, and
  // the masks are selects, so one LDS round trip serves the tile.
#pragma unroll
  for (int m = 0; m < kM / 2; ++m) {
    const int u = wave + 8 * m;
    if (u < ngram) {
      const int kt = u % (NP / 16), rt = u / (NP / 16);
      const bool query = rt < NP / 16;
      const int i = 16 * kt + lr;
      const int t0 = 16 * rt + 4 * lg - (query ? 0 : NP);
      const int zi = s_zc[i], ei = s_ex[i];
      const float rmi = s_rmant[i];
      uint64_t at[4];
      int zt[4], et[4];
      float mt[4], bt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        at[r] = s_anc[t0 + r];
        zt[r] = s_zc[t0 + r];
        et[r] = s_ex[t0 + r];
        mt[r] = s_mant[t0 + r];
        bt[r] = query ? 1.0f : s_beta[t0 + r];
      }
      float* dst = query ? s_y : s_x;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + r;
        // gamma_t / gamma_i: the gates strictly below i down to t, 0 past a zero gate
        const float ratio = t == i ? 1.0f : (zt[r] != zi ? 0.0f : ldexpf(mt[r] * rmi, et[r] - ei));
        const bool keep = t < N && i < N && ((at[r] >> i) & 1ull) && (query || i != t);
        dst[t * MP + i] = keep ? bt[r] * ratio * gram[m][r] : 0.0f;
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
  const float* s_m;  // M [NP][MP], left in region 1 by the last step
  {
    const int steps = s_steps;
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
    s_m = bm;  // behind a barrier: the last step's, else the one after X and Y
  }

  // ---- phase 3: [Q; K] S0 on MFMA from registers.  S0 = hi + lo, hi =
  // bf16(S0) (round to nearest even, the hardware conversion) and lo =
  // bf16(S0 - hi).  Node tile m < kM / 2 is Q: the product S0^T Q^T leaves lane
  // (lr, lg) node 16 m + lr, columns 16 w + 4 lg + r.  The others are K: K S0
  // with A-row i reading node 4 (i & 3) + (i >> 2) of the tile, which leaves
  // lane (lr, lg) column 16 w + lr of nodes 16 m' + 4 r + lg.
  mbf16x8_t shi[kDk / 32], slo[kDk / 32];
#pragma unroll
  for (int u = 0; u < kDk / 16; ++u) f[u] = quad_transpose(f[u], lr & 3);
#pragma unroll
  for (int ks = 0; ks < kDk / 32; ++ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4& fq = f[2 * ks + (j >> 2)];
      const float x = (j & 3) == 0 ? fq.x : (j & 3) == 1 ? fq.y : (j & 3) == 2 ? fq.z : fq.w;
      const __bf16 hv = static_cast<__bf16>(x);
      shi[ks][j] = hv;
      slo[ks][j] = static_cast<__bf16>(x - static_cast<float>(hv));
    }
  }
  const int kperm = 4 * (lr & 3) + (lr >> 2);
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    qks[m] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
    const int row = 16 * m + (m < kM / 2 ? lr : kperm);
#pragma unroll
    for (int ks = 0; ks < kDk / 32; ++ks) {
      const mbf16x8_t nb = __builtin_bit_cast(mbf16x8_t, *reinterpret_cast<const uint4*>(
                                                             r2 + gswz(row, 2 * (32 * ks + 8 * lg))));
      if (m < kM / 2) {
        qks[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(slo[ks], nb, qks[m], 0, 0, 0);
        qks[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(shi[ks], nb, qks[m], 0, 0, 0);
      } else {
        qks[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nb, slo[ks], qks[m], 0, 0, 0);
        qks[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nb, shi[ks], qks[m], 0, 0, 0);
      }
    }
  }

  // ---- phase 4: right-hand side beta_t (v_t - gamma_t (K S0)_t) in
  // registers, lane (lr, lg) holding column 16 w + lr of node 4 ks + lg for
  // k-step ks of the output product.  Rows past N have zero V, K and beta.
  constexpr int nt = NP / 16;
  float rhs[NP / 4];
#pragma unroll
  for (int mt = 0; mt < nt; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 16 * mt + 4 * r + lg;
      rhs[4 * mt + r] = s_beta[n] * (s_u[n * kHUP + 16 * wave + lr] - s_gam[n] * qks[nt + mt][r]);
    }
  }

  // ---- phase 5: O^T = (right-hand side)^T M^T + gamma (Q S0)^T, tiles of
  // 16 state columns x 16 nodes; a lane ends with 4 consecutive columns of
  // one node's output
#pragma unroll
  for (int mm = 0; mm < nt; ++mm) {
    {
      const int ct = wave;
      const int t = 16 * mm + lr;
      const float gt = s_gam[t];
      // M is lower triangular: nodes past this tile do not contribute
      mf32x4_t acc = gt * qks[mm], acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4 * mm + 4; ks += 2) {
        const float bv = s_m[t * MP + 4 * ks + lg];
        const float bv2 = s_m[t * MP + 4 * ks + 4 + lg];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(rhs[ks], bv, acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(rhs[ks + 1], bv2, acc2, 0, 0, 0);
      }
      acc += acc2;
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

// ---------------------------------------------------------------------------
// bf16 inputs, 32 < N <= 128 (see TV_GDN_TRI_FROM).  One 8-wave workgroup
// per (sequence, head), wave w owning state columns 16 w .. 16 w + 15; the
// node count is padded to NP = 16 NT, NT even (64, 96 or 128 nodes; 32 when
// the threshold is lowered).  The Gram products and the solve run
// once per head.
//
//  1. q and k rows (bf16, exact) into LDS; v of this wave's columns into
//     registers in 16-byte pieces (parked in LDS once the solve is done), and
//     after the Gram tiles S0's columns of this wave, in flight through steps
//     2-4, which do not need them.
//  2. Gate products per node, then the Gram tiles [Q; K] K^T on bf16 MFMA,
//     only the 16 x 16 tiles on or below the block diagonal (ancestors precede
//     descendants), each masked and scaled by the gate ratios as it comes out:
//     Y in LDS in fp32, X transposed in bf16 hi and lo parts.  A wave forms
//     the tiles of two block rows (one of Y's parts or X's), reading each
//     row's operands once.
//  3. Diagonal blocks D_b = (I + X_bb)^-1, formed by the wave that formed
//     X_bb, right after its block row (no barrier).  X_bb couples a node only
//     to its strict ancestors inside the block, so X_bb^h = 0 for chains of
//     at most h nodes and the inverse is the product of (I + (-X_bb)^(2^j)),
//     j < ceil(log2 h): at most four steps, each two 16 x 16 fp32 MFMA
//     products; D_b goes where X_bb would, in X's hi/lo form.
//  4. M = Y (I + X)^-1, one block row per wave (a row of M needs only its row
//     of Y and X): M_ta = (Y_ta - sum_{a < c <= t} M_tc X_ca) D_a, each
//     product three bf16 MFMAs on hi/lo parts (about 16 mantissa bits), the
//     row's partial sums in fp32 registers.  M goes over Y as bf16 hi and lo
//     parts.
//  5. [Q; K] S0 on bf16 MFMA from registers, S0 split into hi = bf16(S0) and
//     lo = bf16(S0 - hi) (two products: ~16 mantissa bits): Q S0 transposed,
//     as the output accumulates; K S0 with permuted node rows, which leaves
//     the right-hand side in the output product's operand layout.
//  6. Right-hand side beta (V - gamma K S0) in registers, split into bf16 hi
//     and lo parts, then O = gamma Q S0 + M RHS on bf16 MFMA over 32-node
//     chunks of M's lower-triangular tiles (three products each), and the
//     store.  No barrier after step 4.
// ---------------------------------------------------------------------------

constexpr int kTThreads = 512;

// element (r, c) of a 16 x 16 fp32 tile: row-major, column XOR-swizzled by row
__device__ __forceinline__ int tix(int r, int c) { return r * 16 + (c ^ r); }

// lower-block-triangular tile (rt, kt), kt <= rt
__device__ __forceinline__ int ltri(int rt, int kt) { return rt * (rt + 1) / 2 + kt; }

template <int NT>
struct GdnLds {
  static constexpr int NP = 16 * NT;
  static constexpr int NTRI = NT * (NT + 1) / 2;
  static constexpr int W = (NP + 63) / 64;
  static constexpr int kQK = 2 * NP * kRowB;               // [Q; K] bf16
  static constexpr int kTiles = NTRI * 256 * 4;            // X or Y tiles
  static constexpr int kScr = (kTThreads / 64) * 2 * 256 * 4;  // per wave: two 16 x 16 fp32 tiles
  static constexpr int kSmall = NP * 16 + NP * 4 * 3 + NP * W * 8;  // gate product, alpha, beta, gamma; anc
  static constexpr int kBytes = kQK + 2 * kTiles + kScr + kSmall;
};

// 16 x 16 x 16 fp32 product on v_mfma_f32_16x16x4f32: acc += (sa A) B
__device__ __forceinline__ gf32x4_t mm16(const float* A, const float* B, gf32x4_t acc, int lr, int lg,
                                         float sa = 1.0f) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const float a = sa * A[tix(lr, 4 * ks + lg)];
    const float b = B[tix(4 * ks + lg, lr)];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
  return acc;
}

// a tile in the accumulator layout: lane (lr, lg) holds rows 4 lg .. 4 lg + 3 of column lr
__device__ __forceinline__ gf32x4_t tload(const float* T, int lr, int lg) {
  return gf32x4_t{T[tix(4 * lg, lr)], T[tix(4 * lg + 1, lr)], T[tix(4 * lg + 2, lr)], T[tix(4 * lg + 3, lr)]};
}

__device__ __forceinline__ void tstore(float* T, gf32x4_t v, int lr, int lg) {
#pragma unroll
  for (int r = 0; r < 4; ++r) T[tix(4 * lg + r, lr)] = v[r];
}

// LDS written by this wave is read back by other lanes of the same wave: wait
// for the wave's LDS operations only (global loads stay in flight)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef short gs16x4_t __attribute__((ext_vector_type(4)));

// bf16 hi and lo parts of four fp32 values: hi = bf16(x) (round to nearest
// even), lo = bf16(x - hi); hi + lo carries x to about 16 mantissa bits
__device__ __forceinline__ void split_hilo(gf32x4_t x, gs16x4_t& hi, gs16x4_t& lo) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const __bf16 h = static_cast<__bf16>(x[j]);
    hi[j] = __builtin_bit_cast(short, h);
    lo[j] = __builtin_bit_cast(short, static_cast<__bf16>(x[j] - static_cast<float>(h)));
  }
}

// 16 x 16 x 16 product of hi/lo parts on bf16 MFMA (hi hi + hi lo + lo hi):
// acc += A B, lane (lr, lg) giving A[lr][4 lg + j] and B[4 lg + j][lr]
__device__ __forceinline__ gf32x4_t mm16_hilo(gs16x4_t ah, gs16x4_t al, gs16x4_t bh, gs16x4_t bl, gf32x4_t acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
}

// A 16 x 16 tile of X (or of a diagonal inverse D) kept transposed as the A
// operand of mm16_hilo: bf16 hi part at byte 0, lo part at byte 512, element
// (r, c) of the transpose at r * 32 + c * 2.  Lane (lr, lg) reads or writes
// the four elements (lr, 4 lg .. 4 lg + 3) = the tile's (4 lg + j, lr), which
// is also where an accumulator holds them.
__device__ __forceinline__ void at_read(const unsigned char* t, int lr, int lg, gs16x4_t& hi, gs16x4_t& lo) {
  hi = *reinterpret_cast<const gs16x4_t*>(t + lr * 32 + lg * 8);
  lo = *reinterpret_cast<const gs16x4_t*>(t + 512 + lr * 32 + lg * 8);
}
__device__ __forceinline__ void at_write(unsigned char* t, int lr, int lg, gf32x4_t x) {
  gs16x4_t hi, lo;
  split_hilo(x, hi, lo);
  *reinterpret_cast<gs16x4_t*>(t + lr * 32 + lg * 8) = hi;
  *reinterpret_cast<gs16x4_t*>(t + 512 + lr * 32 + lg * 8) = lo;
}

// Workgroup barrier over LDS only: unlike __syncthreads it does not wait for
// the wave's outstanding global loads, so S0's loads stay in flight across it
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// Byte offset of element (r, c) in the bf16 hi or lo half of a 16 x 16 tile of
// M: row-major, the two 16-byte halves of a row exchanged in rows 8-15, so
// that 16 lanes reading one half of each of 16 rows spread over the banks.
__device__ __forceinline__ int mbyte(int r, int c) { return r * 32 + (((c >> 3) ^ (r >> 3)) << 4) + (c & 7) * 2; }

// Block row T of M = Y (I + X)^-1 (step 4 of the kernel below), with T a
// compile-time constant so that the row's steps are straight-line code.
// accT[a] = (Y_Ta - sum_{c > a} M_Tc X_ca)^T in registers (fp32, the
// accumulator layout, which is also the B-operand layout of mm16_hilo); for c
// from T down, M_Tc^T = D_c^T accT[c] is stored over Y_Tc as bf16 hi and lo
// parts of M_Tc (the output product's operands), then accT[a] -= X_ca^T
// M_Tc^T for every a < c.  X and D are read as transposed hi/lo tiles.
template <int T>
__device__ __forceinline__ void gdn_row_solve(float* r_y, const unsigned char* r_xt, int lr, int lg) {
  float* yrow = r_y + ltri(T, 0) * 256;  // the row's tiles lie one after another
  gf32x4_t accT[T + 1];
#pragma unroll
  for (int a = 0; a <= T; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) accT[a][j] = yrow[a * 256 + tix(lr, 4 * lg + j)];
#pragma unroll
  for (int c = T; c >= 0; --c) {
    gs16x4_t bh, bl, dh, dl;
    split_hilo(accT[c], bh, bl);
    at_read(r_xt + ltri(c, c) * 1024, lr, lg, dh, dl);
    const gf32x4_t mt = mm16_hilo(dh, dl, bh, bl, gf32x4_t{0.f, 0.f, 0.f, 0.f});
    // M_Tc[lr][4 lg + j] in bf16 hi and lo parts for the output product
    mbf16x4_t mh, ml;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mh[j] = static_cast<__bf16>(mt[j]);
      ml[j] = static_cast<__bf16>(mt[j] - static_cast<float>(mh[j]));
    }
    unsigned char* tb = reinterpret_cast<unsigned char*>(yrow + c * 256);
    *reinterpret_cast<uint2*>(tb + mbyte(lr, 4 * lg)) = __builtin_bit_cast(uint2, mh);
    *reinterpret_cast<uint2*>(tb + 512 + mbyte(lr, 4 * lg)) = __builtin_bit_cast(uint2, ml);
    if (c > 0) {
      gs16x4_t nh, nl;  // -M_Tc^T, the updates' B operand
      split_hilo(-mt, nh, nl);
#pragma unroll
      for (int a = 0; a < c; ++a) {
        gs16x4_t xh, xl;
        at_read(r_xt + ltri(c, a) * 1024, lr, lg, xh, xl);
        accT[a] = mm16_hilo(xh, xl, nh, nl, accT[a]);
      }
    }
  }
}

// the wave-uniform row t (or none, t < 0) to its specialised path
template <int NT, int K = 0>
__device__ __forceinline__ void gdn_row_solve_pick(int t, float* r_y, const unsigned char* r_xt, int lr, int lg) {
  if constexpr (K < NT) {
    if (t == K)
      gdn_row_solve<K>(r_y, r_xt, lr, lg);
    else
      gdn_row_solve_pick<NT, K + 1>(t, r_y, r_xt, lr, lg);
  }
}

template <typename TO, int NT, int kOcc>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(kOcc)))
void gdn_tri_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const float* __restrict__ alpha,
                    const float* __restrict__ beta, const float* __restrict__ S0,
                    const uint64_t* __restrict__ anc, int N, int H, TO* __restrict__ out) {
  using L = GdnLds<NT>;
  constexpr int NP = L::NP, NTRI = L::NTRI, W = L::W;
  constexpr int kWaves = kTThreads / 64;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* r_qk = smem;
  float* r_y = reinterpret_cast<float*>(smem + L::kQK);
  float* r_x = r_y + NTRI * 256;
  float* r_s = r_x + NTRI * 256;                                    // scratch tiles
  // X's tiles (and the diagonal inverses over them) transposed in bf16 hi/lo parts
  unsigned char* r_xt = reinterpret_cast<unsigned char*>(r_x);
  // once the solve is done, X and the scratch tiles hold v for the right-hand
  // side: wave w's 16 columns of every node, 32 bytes per node
  uint16_t* r_v = reinterpret_cast<uint16_t*>(r_x);
  static_assert(NTRI * 1024 + kWaves * 2048 >= NP * 32 * kWaves, "v fits X and the scratch tiles");
  static_assert(NT % 2 == 0, "node tiles come in pairs (32-node chunks of the output product)");
  float4* s_gp = reinterpret_cast<float4*>(r_s + kWaves * 512);     // [NP] (mant, 1/mant, zeros, exponent)
  float* s_alpha = reinterpret_cast<float*>(s_gp + NP);
  float* s_beta = s_alpha + NP;
  float* s_gam = s_beta + NP;
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(s_gam + NP);  // [NP][W]
  __shared__ int s_maxdepth;

  const int bh = blockIdx.x;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // lane (lr, lg) owns state column col = 16 wave + lr

  // ---- 1. loads: the per-node gates and ancestor words first, then q and k
  // rows into LDS, then v of this wave's columns, which stays in flight
  if (tid == 0) s_maxdepth = 1;
  float g_a = 1.0f, g_b = 0.0f;
  uint64_t g_w[W];
#pragma unroll
  for (int w = 0; w < W; ++w) g_w[w] = 0ull;
  if (tid < N) {
    const size_t nh = (static_cast<size_t>(b) * N + tid) * H + h;
    g_a = alpha[nh];
    g_b = beta[nh];
#pragma unroll
    for (int w = 0; w < W; ++w) g_w[w] = anc[(static_cast<size_t>(b) * N + tid) * W + w];
  }
  constexpr int kGr = 2 * NP * (kRowB / 16);  // 16-byte granules of [Q; K]
  constexpr int kPer = (kGr + kTThreads - 1) / kTThreads;
  uint4 g[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = tid + u * kTThreads;
    const int row = e >> 4, gr = e & 15;
    const bool isk = row >= NP;
    const int t = isk ? row - NP : row;
    g[u] = make_uint4(0, 0, 0, 0);
    if (e < kGr && t < N)
      g[u] = *reinterpret_cast<const uint4*>((isk ? k : q) +
                                             ((static_cast<size_t>(b) * N + t) * H + h) * kDk + gr * 8);
  }
  // v of this wave's columns, 16 bytes (8 columns of one node) per load:
  // granule e = lane + 64 u is node e / 2, columns 16 w + 8 (e % 2) .. + 7.
  // Nodes past N read node N - 1 and are zeroed when v is parked: loads
  // under a condition would be waited for at once (their registers join
  // the zero default's), and v is to stay in flight through steps 2-4.
  constexpr int kVPer = (2 * NP + 63) / 64;
  uint4 vg[kVPer];
#pragma unroll
  for (int u = 0; u < kVPer; ++u) {
    const int e = lane + 64 * u, t = min(e >> 1, N - 1);
    vg[u] = *reinterpret_cast<const uint4*>(v + ((static_cast<size_t>(b) * N + t) * H + h) * kDk + 16 * wave +
                                            8 * (e & 1));
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = tid + u * kTThreads;
    if (e < kGr) *reinterpret_cast<uint4*>(r_qk + gswz(e >> 4, (e & 15) * 16)) = g[u];
  }
  if (tid < NP) {
    s_alpha[tid] = g_a;
    s_beta[tid] = g_b;
#pragma unroll
    for (int w = 0; w < W; ++w) s_anc[tid * W + w] = tid < N ? anc_clean(g_w[w], tid, w) : 0ull;
  }
  lds_barrier();

  // ---- 2. gate products per node, four lanes per node: lane q of a quad
  // takes the ancestors in nodes 32 q .. 32 q + 31 (zero count, mantissa and
  // exponent, factors in node order), and the quad combines its four parts;
  // then the masked Gram tiles
  {
    const int t = tid >> 2, qd = tid & 3;
    int zeros = 0, ex = 0, dpt = 0;
    float mant = 1.0f;
    if (t < NP) {
      // (a quarter past the node words holds no node)
      uint32_t m = (qd >> 1) < W ? static_cast<uint32_t>(s_anc[t * W + (qd >> 1)] >> (32 * (qd & 1))) : 0u;
      dpt = __popc(m);
      while (m) {
        const float al = s_alpha[32 * qd + __ffs(m) - 1];
        m &= m - 1;
        if (al == 0.0f) {
          ++zeros;
        } else {
          int ea, em;
          mant *= frexpf(al, &ea);
          mant = frexpf(mant, &em);
          ex += ea + em;
        }
      }
    }
    // parts 0 and 1, 2 and 3, then the two pairs
    {
      const float om = quad_dpp<0xb1>(mant);
      const int oz = __float_as_int(quad_dpp<0xb1>(__int_as_float(zeros)));
      const int oe = __float_as_int(quad_dpp<0xb1>(__int_as_float(ex)));
      const int od = __float_as_int(quad_dpp<0xb1>(__int_as_float(dpt)));
      int em;
      mant = frexpf(mant * om, &em);
      ex += oe + em;
      zeros += oz;
      dpt += od;
    }
    {
      const float om = quad_dpp<0x4e>(mant);
      const int oz = __float_as_int(quad_dpp<0x4e>(__int_as_float(zeros)));
      const int oe = __float_as_int(quad_dpp<0x4e>(__int_as_float(ex)));
      const int od = __float_as_int(quad_dpp<0x4e>(__int_as_float(dpt)));
      int em;
      mant = frexpf(mant * om, &em);
      ex += oe + em;
      zeros += oz;
      dpt += od;
    }
    if (t < NP && qd == 0) {
      s_gam[t] = zeros ? 0.0f : ldexpf(mant, ex);
      s_gp[t] = make_float4(mant, 1.0f / mant, __int_as_float(zeros), __int_as_float(ex));
    }
    // the deepest node of the wave (bit by bit over ballots), one LDS max per wave
    const int d = t < N ? dpt : 0;
    int dm = 0;
#pragma unroll
    for (int bit = 7; bit >= 0; --bit)
      if (__ballot(d >= (dm | (1 << bit)))) dm |= 1 << bit;
    if (lane == 0 && dm > 0) atomicMax(&s_maxdepth, dm);
  }
  lds_barrier();
  // Waves 0-3 form X's tiles, waves 4-7 Y's (X's cost more, the beta factor
  // and the hi/lo stores, and of the two waves of a SIMD the older one runs
  // first, so the pair ends closer together).  Wave p of a part takes the
  // block rows p and NT - 1 - p (NT + 1 tiles: balanced), so a row's A
  // operand (its bf16 q or k rows) and its mask operands are read once for
  // all of the row's tiles; the next tile's key rows are read before the
  // current tile's products.  The masks and gate ratios are selects.
  // (I + X_bb)^-1 of a diagonal block from X_bb in the accumulator layout
  // (lane (lr, lg) holding rows 4 lg .. + 3 of column lr): X_bb couples a node
  // only to its strict ancestors inside the block, so X_bb^h = 0 for chains
  // of at most h nodes and the inverse is the product of (I + (-X_bb)^(2^j)),
  // j < ceil(log2 h), at most four steps of two 16 x 16 fp32 MFMA products,
  // through the wave's two scratch tiles
  const int hmax = min(16, s_maxdepth);
  int J = 1;
  while ((1 << J) < hmax) ++J;
  float* mb = r_s + wave * 512;
  float* pb = mb + 256;
  auto invert_diag = [&](gf32x4_t xv) __attribute__((always_inline)) {
    tstore(mb, xv, lr, lg);
    wave_lds_sync();
    // M = I - X (the first factor), P = X X (the next power)
    const gf32x4_t p = mm16(mb, mb, gf32x4_t{0.f, 0.f, 0.f, 0.f}, lr, lg);
    gf32x4_t mm;
#pragma unroll
    for (int r = 0; r < 4; ++r) mm[r] = (4 * lg + r == lr ? 1.0f : 0.0f) - xv[r];
    wave_lds_sync();
    tstore(mb, mm, lr, lg);
    tstore(pb, p, lr, lg);
    wave_lds_sync();
    for (int j = 1; j < J; ++j) {
      // M <- M + M P, and P <- P P for the next step
      const gf32x4_t m2 = mm16(mb, pb, tload(mb, lr, lg), lr, lg);
      gf32x4_t p2 = p;
      if (j + 1 < J) p2 = mm16(pb, pb, gf32x4_t{0.f, 0.f, 0.f, 0.f}, lr, lg);
      wave_lds_sync();
      tstore(mb, m2, lr, lg);
      if (j + 1 < J) tstore(pb, p2, lr, lg);
      wave_lds_sync();
    }
    return tload(mb, lr, lg);
  };
  {
    const int part = 1 - (wave >> 2), p = wave & 3;
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
      const int rt = hr == 0 ? p : NT - 1 - p;
      if (p < (NT + 1) / 2 && !(hr == 1 && rt == p)) {
        const int arow = (part ? NP : 0) + 16 * rt + lr, t0 = 16 * rt + 4 * lg;
        uint4 a[kDk / 32];
#pragma unroll
        for (int ks = 0; ks < kDk / 32; ++ks)
          a[ks] = *reinterpret_cast<const uint4*>(r_qk + gswz(arow, 2 * (32 * ks + 8 * lg)));
        float4 gt[4];
        uint64_t at[4][W];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gt[r] = s_gp[t0 + r];
#pragma unroll
          for (int w = 0; w < W; ++w) at[r][w] = s_anc[(t0 + r) * W + w];
        }
        const float4 bt = part ? *reinterpret_cast<const float4*>(s_beta + t0) : make_float4(1.f, 1.f, 1.f, 1.f);
        const float bts[4] = {bt.x, bt.y, bt.z, bt.w};
        uint4 bk[2][kDk / 32];
        float4 gi[2];
        auto read_col = [&](int kt, int sl) __attribute__((always_inline)) {
#pragma unroll
          for (int ks = 0; ks < kDk / 32; ++ks)
            bk[sl][ks] = *reinterpret_cast<const uint4*>(r_qk + gswz(NP + 16 * kt + lr, 2 * (32 * ks + 8 * lg)));
          gi[sl] = s_gp[16 * kt + lr];
        };
        read_col(0, 0);
        gf32x4_t diag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
          if (kt <= rt) {
            if (kt + 1 <= rt) read_col(kt + 1, (kt + 1) & 1);
            const int sl = kt & 1;
            gf32x4_t g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < kDk / 32; ++ks)
              g = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(gbf16x8_t, a[ks]),
                                                           __builtin_bit_cast(gbf16x8_t, bk[sl][ks]), g, 0, 0, 0);
            // Y over ancestors-or-self, X over strict ancestors (times beta_t);
            // Y in fp32, X transposed in bf16 hi/lo parts (the operand form of
            // the back-substitution)
            const int i = 16 * kt + lr;
            gf32x4_t val;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = t0 + r;
              uint64_t aw = at[r][0];
#pragma unroll
              for (int w = 1; w < W; ++w) aw = (kt >> 2) == w ? at[r][w] : aw;
              const bool on = ((aw >> (i & 63)) & 1ull) && !(part && i == t);
              // gamma_t / gamma_i: 0 when the path below i holds a zero gate
              float ratio = __builtin_amdgcn_ldexpf(gt[r].x * gi[sl].y,
                                                    __float_as_int(gt[r].w) - __float_as_int(gi[sl].w));
              ratio = __float_as_int(gt[r].z) != __float_as_int(gi[sl].z) ? 0.0f : ratio;
              ratio = i == t ? 1.0f : ratio;
              val[r] = on ? bts[r] * ratio * g[r] : 0.0f;
            }
            if (part) {
              if (kt == rt)
                diag = val;  // inverted below, after the row
              else
                at_write(r_xt + ltri(rt, kt) * 1024, lr, lg, val);
            } else {
              float* dst = r_y + ltri(rt, kt) * 256;
#pragma unroll
              for (int r = 0; r < 4; ++r) dst[tix(4 * lg + r, lr)] = val[r];
            }
          }
        }
        // X's diagonal tile becomes D_rt = (I + X_rt,rt)^-1, in the same
        // transposed hi/lo form, right here: no other wave needs X_rt,rt
        if (part) at_write(r_xt + ltri(rt, rt) * 1024, lr, lg, invert_diag(diag));
      }
    }
  }
  // S0 goes out once the Gram tiles are formed and stays in flight through
  // steps 3 and 4, which do not need it (issued before the gate products it
  // was no faster).  S0 of this wave's columns in 16-byte loads: load
  // u = 2 ks + hf gives lane (lr, lg) = (4 q + b, lg) columns 16 w + 4 q ..
  // + 3 of row 32 ks + 8 lg + 4 hf + b; a 4 x 4 transpose inside each quad
  // (in step 5) then leaves lane (lr, lg) rows 32 ks + 8 lg .. + 7 of column
  // `col`, the bf16 operand layout
  float4 s0q[kDk / 16];
  {
    const float* s0 = S0 + static_cast<size_t>(bh) * kDk * kDk + 16 * wave + 4 * (lr >> 2);
#pragma unroll
    for (int u = 0; u < kDk / 16; ++u)
      s0q[u] = *reinterpret_cast<const float4*>(s0 + (32 * (u >> 1) + 8 * lg + 4 * (u & 1) + (lr & 3)) * kDk);
  }
  lds_barrier();

  // ---- 4. M = Y (I + X)^-1 by block rows: row t of M depends only on row t
  // of Y and on X, so each wave takes one block row (gdn_row_solve) and no
  // barrier is needed until the rows are done.  Inside a row the products are
  // right-looking and transposed, so that the updates of one step do not
  // depend on one another, and an accumulator feeds the next product as its
  // B operand straight from registers.  Waves w and w + 4 take rows
  // NT - 1 - w and w, which balances the SIMD that the two waves share when
  // waves are dealt to SIMDs in turn.
  {
    const int t = wave < 4 ? NT - 1 - wave : (wave - 4 < NT - 4 ? wave - 4 : -1);
    gdn_row_solve_pick<NT>(t, r_y, r_xt, lr, lg);
  }
  // ---- 5. [Q; K] S0 for this wave's columns, right after its block row (a
  // wave whose row is short forms them while the longer row of the other
  // wave on its SIMD is still running its chain of dependent products; they
  // read only the q and k rows).  Node tile mt of Q: the product
  // S0^T Q^T leaves lane (lr, lg) node 16 mt + lr, columns 16 w + 4 lg + r.  Of
  // K: K S0 with A-row i of tile mt reading node 32 (mt / 2) + 8 (i / 4) +
  // 4 (mt % 2) + i % 4, which leaves lane (lr, lg) column `col` of nodes
  // 32 c + 8 lg + j, j < 8, in tiles 2c and 2c + 1: the A-operand layout of
  // the output product over 32-node chunks.
  gbf16x8_t shi[kDk / 32], slo[kDk / 32];
#pragma unroll
  for (int u = 0; u < kDk / 16; ++u) s0q[u] = quad_transpose(s0q[u], lr & 3);
#pragma unroll
  for (int ks = 0; ks < kDk / 32; ++ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4& fq = s0q[2 * ks + (j >> 2)];
      const float x = (j & 3) == 0 ? fq.x : (j & 3) == 1 ? fq.y : (j & 3) == 2 ? fq.z : fq.w;
      const __bf16 hv = static_cast<__bf16>(x);
      shi[ks][j] = hv;
      slo[ks][j] = static_cast<__bf16>(x - static_cast<float>(hv));
    }
  }
  gf32x4_t qs[NT], ksa[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    qs[mt] = gf32x4_t{0.f, 0.f, 0.f, 0.f};
    ksa[mt] = gf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDk / 32; ++ks) {
      const gbf16x8_t q8 = __builtin_bit_cast(
          gbf16x8_t, *reinterpret_cast<const uint4*>(r_qk + gswz(16 * mt + lr, 2 * (32 * ks + 8 * lg))));
      const int knode = 32 * (mt >> 1) + 8 * (lr >> 2) + 4 * (mt & 1) + (lr & 3);
      const gbf16x8_t k8 = __builtin_bit_cast(
          gbf16x8_t, *reinterpret_cast<const uint4*>(r_qk + gswz(NP + knode, 2 * (32 * ks + 8 * lg))));
      qs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(slo[ks], q8, qs[mt], 0, 0, 0);
      qs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(shi[ks], q8, qs[mt], 0, 0, 0);
      ksa[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k8, slo[ks], ksa[mt], 0, 0, 0);
      ksa[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k8, shi[ks], ksa[mt], 0, 0, 0);
    }
  }

  lds_barrier();  // every block row of M is done, X is free
  // v into this wave's part of X and the scratch tiles (free since the
  // barrier above); only this wave reads it back
  uint16_t* vw = r_v + wave * NP * 16;
#pragma unroll
  for (int u = 0; u < kVPer; ++u) {
    const int e = lane + 64 * u;
    if (e < 2 * NP)
      *reinterpret_cast<uint4*>(vw + (e >> 1) * 16 + 8 * (e & 1)) = (e >> 1) < N ? vg[u] : make_uint4(0, 0, 0, 0);
  }

  // ---- 6. right-hand side RHS = beta (V - gamma K S0) in registers, split
  // into bf16 hi and lo parts: lane (lr, lg) holds column `col` of nodes
  // 32 c + 8 lg + j of chunk c (rows past N have zero v, k and beta).  Then
  // O^T = RHS^T M^T + gamma (Q S0)^T on bf16 MFMA over 32-node chunks of M's
  // lower-triangular tiles, three products per chunk (hi hi, hi lo, lo hi:
  // about 16 mantissa bits), a lane ending with four consecutive columns of
  // one node
  wave_lds_sync();  // this wave's v is in LDS
  constexpr int NH = NT / 2;
  gbf16x8_t rh[NH], rl[NH];
#pragma unroll
  for (int c = 0; c < NH; ++c) {
    const int n0 = 32 * c + 8 * lg;
    const float4 b0 = *reinterpret_cast<const float4*>(s_beta + n0);
    const float4 b1 = *reinterpret_cast<const float4*>(s_beta + n0 + 4);
    const float4 g0 = *reinterpret_cast<const float4*>(s_gam + n0);
    const float4 g1 = *reinterpret_cast<const float4*>(s_gam + n0 + 4);
    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float ks0 = j < 4 ? ksa[2 * c][j & 3] : ksa[2 * c + 1][j & 3];
      const float x = bv[j] * (bf16_to_f32(vw[(n0 + j) * 16 + lr]) - gv[j] * ks0);
      const __bf16 hv = static_cast<__bf16>(x);
      rh[c][j] = hv;
      rl[c][j] = static_cast<__bf16>(x - static_cast<float>(hv));
    }
  }
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const int t = 16 * rt + lr;
    gf32x4_t acc = s_gam[t] * qs[rt], acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NH; ++c) {
      if (2 * c <= rt) {
        // lane (lr, lg): row t, nodes 32 c + 8 lg .. + 7 of tile 2c + lg / 2,
        // none past the diagonal tile
        const int a = 2 * c + (lg >> 1);
        const unsigned char* tb = reinterpret_cast<const unsigned char*>(r_y + ltri(rt, a <= rt ? a : rt) * 256);
        uint4 mh = *reinterpret_cast<const uint4*>(tb + mbyte(lr, 8 * (lg & 1)));
        uint4 ml = *reinterpret_cast<const uint4*>(tb + 512 + mbyte(lr, 8 * (lg & 1)));
        if (2 * c + 1 > rt && a > rt) mh = ml = make_uint4(0, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh[c], __builtin_bit_cast(gbf16x8_t, mh), acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rh[c], __builtin_bit_cast(gbf16x8_t, ml), acc2, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rl[c], __builtin_bit_cast(gbf16x8_t, mh), acc2, 0, 0, 0);
      }
    }
    acc += acc2;
    if (t < N) {
      const size_t off = ((static_cast<size_t>(b) * N + t) * H + h) * kDk + 16 * wave + 4 * lg;
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

// ---------------------------------------------------------------------------
// fp32 inputs.  One 256-thread workgroup per (sequence, head, 32 state
// columns), every product as fp32 FMAs: the gate products, X and Y over the
// ancestor pairs (packed lower triangle, diagonal included), K S0 and Q S0
// for the column block, then forward substitution one depth level at a time
// and the outputs.  q and k rows are read through the caches, not staged.
// ---------------------------------------------------------------------------

size_t gdn_f32_lds_bytes(int N, int W) {
  const size_t P = static_cast<size_t>(N) * (N + 1) / 2;
  // S0 block; X, Y; U, K S0, Q S0; gamma, beta; depth; anc
  return sizeof(float) * (static_cast<size_t>(kDk) * kGC + 2 * P + 3 * static_cast<size_t>(N) * kGC + 2 * N) +
         sizeof(int) * N + sizeof(uint64_t) * N * W + 16;
}

__device__ __forceinline__ float dot128(const float* a, const float* b) {
  float s = 0.0f;
#pragma unroll 8
  for (int d = 0; d < kDk; d += 4) {
    const float4 x = *reinterpret_cast<const float4*>(a + d);
    const float4 y = *reinterpret_cast<const float4*>(b + d);
    s = fmaf(x.x, y.x, fmaf(x.y, y.y, fmaf(x.z, y.z, fmaf(x.w, y.w, s))));
  }
  return s;
}

__global__ __launch_bounds__(kGThreads) void gdn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ S0,
    const uint64_t* __restrict__ anc, int N, int W, int H, int BH, float* __restrict__ out) {
  extern __shared__ __align__(16) float lds[];
  const int P = N * (N + 1) / 2;
  float* s_s0 = lds;              // [kDk][kGC]
  float* s_x = s_s0 + kDk * kGC;  // packed: (t, i) at t (t + 1) / 2 + i
  float* s_y = s_x + P;
  float* s_u = s_y + P;           // [N][kGC]  V, then the right-hand side, then U
  float* s_ks = s_u + N * kGC;    // [N][kGC]  K S0
  float* s_qs = s_ks + N * kGC;   // [N][kGC]  Q S0
  float* s_gam = s_qs + N * kGC;  // [N]
  float* s_beta = s_gam + N;      // [N]
  int* s_depth = reinterpret_cast<int*>(s_beta + N);
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(
      (reinterpret_cast<uintptr_t>(s_depth + N) + 7) & ~static_cast<uintptr_t>(7));  // [N][W]
  __shared__ int s_maxdepth;
  __shared__ float s_alpha[TV_MAX_NODES];

  int bh, cb;
  if (!gdn_block(blockIdx.x, BH, kNCB, &bh, &cb)) return;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x;
  const int col0 = cb * kGC;
  const size_t row0 = static_cast<size_t>(b) * N;  // node rows of this sequence

  if (tid == 0) s_maxdepth = 1;
  for (int t = tid; t < N; t += kGThreads) {
    const size_t nh = (row0 + t) * H + h;
    s_alpha[t] = alpha[nh];
    s_beta[t] = beta[nh];
    for (int w = 0; w < W; ++w) s_anc[t * W + w] = anc_clean(anc[(row0 + t) * W + w], t, w);
  }
  {
    const float* s0 = S0 + static_cast<size_t>(bh) * kDk * kDk + col0;
    for (int e = tid; e < kDk * kGC / 4; e += kGThreads) {
      const int d = e / (kGC / 4), c4 = e % (kGC / 4);
      reinterpret_cast<float4*>(s_s0)[e] =
          *reinterpret_cast<const float4*>(s0 + static_cast<size_t>(d) * kDk + 4 * c4);
    }
  }
  __syncthreads();

  // gamma (a direct product: exactly 0 past a zero gate) and depth per node
  for (int t = tid; t < N; t += kGThreads) {
    float gm = 1.0f;
    int dpt = 0;
    for (int w = 0; w < W; ++w) {
      uint64_t m = s_anc[t * W + w];
      dpt += __popcll(m);
      while (m) {
        gm *= s_alpha[64 * w + __ffsll(static_cast<unsigned long long>(m)) - 1];
        m &= m - 1;
      }
    }
    s_gam[t] = gm;
    s_depth[t] = dpt;
    atomicMax(&s_maxdepth, dpt);
  }
  // X and Y over the pairs (t, i <= t)
  for (int p = tid; p < P; p += kGThreads) {
    int t = static_cast<int>((sqrtf(8.0f * p + 1.0f) - 1.0f) * 0.5f);
    while (t * (t + 1) / 2 > p) --t;
    while ((t + 1) * (t + 2) / 2 <= p) ++t;
    const int i = p - t * (t + 1) / 2;
    float xv = 0.0f, yv = 0.0f;
    if ((s_anc[t * W + (i >> 6)] >> (i & 63)) & 1ull) {
      // product of the gates on t's path strictly below i
      float r = 1.0f;
      for (int w = 0; w < W; ++w) {
        uint64_t seg = s_anc[t * W + w] & ~s_anc[i * W + w];
        while (seg) {
          r *= s_alpha[64 * w + __ffsll(static_cast<unsigned long long>(seg)) - 1];
          seg &= seg - 1;
        }
      }
      const float* ki = k + ((row0 + i) * H + h) * kDk;
      yv = r * dot128(q + ((row0 + t) * H + h) * kDk, ki);
      if (i != t) xv = s_beta[t] * r * dot128(k + ((row0 + t) * H + h) * kDk, ki);
    }
    s_x[p] = xv;
    s_y[p] = yv;
  }
  // K S0 and Q S0 for the column block, and V: thread = (column c, node group)
  {
    constexpr int kGroups = kGThreads / kGC;
    const int c = tid % kGC, grp = tid / kGC;
    for (int t = grp; t < N; t += kGroups) {
      const float* kt = k + ((row0 + t) * H + h) * kDk;
      const float* qt = q + ((row0 + t) * H + h) * kDk;
      float ak = 0.0f, aq = 0.0f;
#pragma unroll 4
      for (int d = 0; d < kDk; d += 4) {
        const float4 kv4 = *reinterpret_cast<const float4*>(kt + d);
        const float4 qv4 = *reinterpret_cast<const float4*>(qt + d);
        const float s0a = s_s0[(d + 0) * kGC + c], s0b = s_s0[(d + 1) * kGC + c];
        const float s0c = s_s0[(d + 2) * kGC + c], s0d = s_s0[(d + 3) * kGC + c];
        ak = fmaf(kv4.x, s0a, fmaf(kv4.y, s0b, fmaf(kv4.z, s0c, fmaf(kv4.w, s0d, ak))));
        aq = fmaf(qv4.x, s0a, fmaf(qv4.y, s0b, fmaf(qv4.z, s0c, fmaf(qv4.w, s0d, aq))));
      }
      s_ks[t * kGC + c] = ak;
      s_qs[t * kGC + c] = aq;
      s_u[t * kGC + c] = v[((row0 + t) * H + h) * kDk + col0 + c];
    }
  }
  __syncthreads();

  // right-hand side beta_t (v_t - gamma_t (K S0)_t)
  for (int e = tid; e < N * kGC; e += kGThreads) {
    const int t = e / kGC;
    s_u[e] = s_beta[t] * (s_u[e] - s_gam[t] * s_ks[e]);
  }
  __syncthreads();

  // forward substitution, one depth level at a time
  const int maxdepth = s_maxdepth;
  for (int lvl = 2; lvl <= maxdepth; ++lvl) {
    for (int e = tid; e < N * kGC; e += kGThreads) {
      const int t = e / kGC, c = e % kGC;
      if (s_depth[t] != lvl) continue;
      const float* xr = s_x + t * (t + 1) / 2;
      float acc = s_u[e];
      for (int w = 0; w < W; ++w) {
        uint64_t m = s_anc[t * W + w];
        if (t >= 64 * w && t < 64 * w + 64) m &= ~(1ull << (t - 64 * w));
        while (m) {
          const int i = 64 * w + __ffsll(static_cast<unsigned long long>(m)) - 1;
          acc = fmaf(-xr[i], s_u[i * kGC + c], acc);
          m &= m - 1;
        }
      }
      s_u[e] = acc;
    }
    __syncthreads();
  }

  // outputs gamma_t (Q S0)_t + sum over ancestors-or-self of Y U
  for (int e = tid; e < N * kGC; e += kGThreads) {
    const int t = e / kGC, c = e % kGC;
    const float* yr = s_y + t * (t + 1) / 2;
    float o = s_gam[t] * s_qs[e];
    for (int w = 0; w < W; ++w) {
      uint64_t m = s_anc[t * W + w];
      while (m) {
        const int i = 64 * w + __ffsll(static_cast<unsigned long long>(m)) - 1;
        o = fmaf(yr[i], s_u[i * kGC + c], o);
        m &= m - 1;
      }
    }
    out[((row0 + t) * H + h) * kDk + col0 + c] = o;
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

template <typename TO, int NT, int kOcc>
hipError_t launch_gdn_tri_occ(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                              int H, void* out, hipStream_t stream) {
  constexpr int lds = GdnLds<NT>::kBytes;
  static_assert(lds + 16 <= 160 * 1024, "LDS budget");
  static_assert(kOcc == 2 || 2 * (lds + 16) <= 160 * 1024, "two workgroups per CU fit the LDS");
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t attr = max_lds_once(lds_set, reinterpret_cast<const void*>(&gdn_tri_kernel<TO, NT, kOcc>), lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gdn_tri_kernel<TO, NT, kOcc>), dim3(static_cast<unsigned>(B) * H), dim3(kTThreads), lds,
                     stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), alpha, beta, S0, anc, N, H, static_cast<TO*>(out));
  return hipGetLastError();
}

// Up to 64 padded nodes the kernel's LDS leaves room for two workgroups per
// CU, and a register budget of 128 (four waves per SIMD, a few spilled
// registers) lets them run together: faster once the grid has more
// workgroups than CUs (B = 32, H = 16, 40 nodes: 22.0 against 25.0 us), slower
// when every workgroup has a CU to itself (B = 16: 14.4 against 13.1 us).
template <typename TO, int NT>
hipError_t launch_gdn_tri_nt(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                             int H, void* out, hipStream_t stream) {
  if constexpr (NT <= 4) {
    if (static_cast<long long>(B) * H > device_cus())
      return launch_gdn_tri_occ<TO, NT, 4>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
  }
  return launch_gdn_tri_occ<TO, NT, 2>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
}

// A grid that fits the CUs one workgroup each asks for more LDS than half a
// CU's, so that no two of its workgroups share a CU.
constexpr size_t kGdnSpreadLds = 81 * 1024;

template <typename TO, int kM>
hipError_t launch_gdn_head_m(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                             int H, void* out, hipStream_t stream) {
  const size_t most = gdn_mfma_lds_bytes(8 * kM);
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t attr = max_lds_once(lds_set, reinterpret_cast<const void*>(&gdn_head_kernel<TO, kM>),
                                       static_cast<int>(most > kGdnSpreadLds ? most : kGdnSpreadLds));
  if (attr != hipSuccess) return attr;
  size_t lds = gdn_mfma_lds_bytes(N);
  if (static_cast<long long>(B) * H <= device_cus() && lds < kGdnSpreadLds) lds = kGdnSpreadLds;
  hipLaunchKernelGGL((gdn_head_kernel<TO, kM>), dim3(static_cast<unsigned>(B) * H), dim3(kMThreads),
                     lds, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), alpha, beta, S0,
                     anc, N, H, static_cast<TO*>(out));
  return hipGetLastError();
}

template <typename TO>
hipError_t launch_gdn_head(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                           int H, void* out, hipStream_t stream) {
  switch ((N + 15) / 16) {
    case 1: return launch_gdn_head_m<TO, 2>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    case 2: return launch_gdn_head_m<TO, 4>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    case 3: return launch_gdn_head_m<TO, 6>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    case 4: return launch_gdn_head_m<TO, 8>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename TO>
hipError_t launch_gdn_tri(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                           int H, void* out, hipStream_t stream) {
#define TV_GDN_NT(X, NT) \
  case X: return launch_gdn_tri_nt<TO, NT>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream)
  switch ((N + 31) / 32) {  // node tiles in pairs: the output product takes 32 nodes per step
    TV_GDN_NT(1, 2);
    TV_GDN_NT(2, 4);
    TV_GDN_NT(3, 6);
    TV_GDN_NT(4, 8);
    default: return hipErrorInvalidValue;
  }
#undef TV_GDN_NT
}

hipError_t launch_gdn_f32(const void* q, const void* k, const void* v, const float* alpha,
                          const float* beta, const float* S0, const uint64_t* anc, int B, int N,
                          int H, void* out, hipStream_t stream) {
  const int W = (N + 63) / 64;
  const size_t lds = gdn_f32_lds_bytes(N, W);
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t attr = max_lds_once(lds_set, reinterpret_cast<const void*>(&gdn_f32_kernel),
                                       static_cast<int>(gdn_f32_lds_bytes(TV_MAX_NODES, (TV_MAX_NODES + 63) / 64)));
  if (attr != hipSuccess) return attr;
  const int BH = B * H;
  hipLaunchKernelGGL(gdn_f32_kernel, dim3(gdn_grid(BH, kNCB)), dim3(kGThreads), lds, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                     alpha, beta, S0, anc, N, W, H, BH, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn(const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* S0, const uint64_t* anc, int B, int N, int H,
                      int Dk, int Dv, tv_dtype dtype, tv_dtype out_dtype, void* out,
                      hipStream_t stream) {
  (void)Dk;
  (void)Dv;
  if (dtype == TV_BF16 && out_dtype == TV_BF16)
    return N < TV_GDN_TRI_FROM ? launch_gdn_head<uint16_t>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream)
                               : launch_gdn_tri<uint16_t>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
  if (dtype == TV_BF16 && out_dtype == TV_F32)
    return N < TV_GDN_TRI_FROM ? launch_gdn_head<float>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream)
                               : launch_gdn_tri<float>(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
  if (dtype == TV_F32 && out_dtype == TV_F32)
    return launch_gdn_f32(q, k, v, alpha, beta, S0, anc, B, N, H, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace tv
