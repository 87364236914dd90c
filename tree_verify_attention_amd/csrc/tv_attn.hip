// Tree-masked attention over a paged context, for gfx950.
//
// Serve-integration spec, section "2. Verify: tree attention mask": each
// draft node attends to every committed context key (the expensive part: a
// stream of the paged KV cache) and, among the nodes, only to its ancestors
// and itself; the mask composes with the layer's sliding window.
//
// Work unit = (sequence b, kv head g, row group, context split).  The query
// tile is the G*N rows (node, query head of the group) that share kv head g,
// 64 rows per workgroup (4 waves x 16 rows).  The split's keys stream through
// a ring of LDS stages, 32 keys per stage, filled by LDS DMA straight from
// HBM (no register staging), several stages in flight while one is computed.
// The split's page indices are cached in LDS first, so no load waits on a
// page-table lookup.
//
// Scores are formed transposed (S^T = K Q^T, K rows as the MFMA A operand
// read straight from the row-major stage) so that each lane's MFMA result
// holds keys of a single query row: the online softmax then needs two
// cross-lane steps per row, and the probabilities feed the P.V MFMA
// (O^T = V^T P^T) straight from registers.  V^T comes out of the row-major
// stage through the LDS transpose read.  Granules of 16 bytes are XOR
// swizzled by row so both operand reads spread over the LDS banks.
//
// The split that holds the end of the context also takes the node keys,
// masked by the ancestor word of each row's node.  A split writes fp32
// partials (acc, m, l); a second kernel merges them by log-sum-exp.  A
// sequence whose keys fit one split writes its output directly.
#include <atomic>

#include "tv_internal.h"

#ifndef TV_ATTN_LDS_BUDGET
#define TV_ATTN_LDS_BUDGET 65536  // bytes of LDS for the K and V rings of a workgroup
#endif
#ifndef TV_ATTN_MIN_WG
#define TV_ATTN_MIN_WG 2  // workgroups per CU the register budget is sized for
#endif

namespace tv {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = kWaves * 16;  // query rows per workgroup
constexpr int kTile = 32;           // keys per LDS stage
constexpr int kThreads = kWaves * 64;
constexpr int kMaxPages = 1024;     // page indices of one stream segment cached in LDS
constexpr int kSplitPages = 4096;   // of one split (splits are capped to fit)
constexpr int kAncW = (TV_MAX_NODES + 63) / 64;  // ancestor words per node at most
static_assert(kThreads >= TV_MAX_NODES, "one thread per node position");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// kTeams teams of kWaves waves share a workgroup: a ring stage holds kTeams
// consecutive 32-key tiles, team i computes the i-th, and the teams' softmax
// states are merged at the end (more waves per CU on short key ranges).
template <typename T, int D, int kTeams = 1>
struct Cfg {
  static constexpr int kEsz = sizeof(T);
  static constexpr int kRowBytes = D * kEsz;           // one key (or value) row
  static constexpr int kGran = kRowBytes / 16;          // 16-byte granules per row
  static constexpr int kSwz = (kGran < 16 ? kGran : 16) - 1;
  static constexpr int kTileBytes = kTile * kRowBytes;  // K (or V) of one tile
  static constexpr int kStageKeys = kTile * kTeams;     // keys per ring stage
  static constexpr int kStageBytes = kTileBytes * kTeams;
  static constexpr int kNW = kWaves * kTeams;           // waves per workgroup
  // K and V of a stage live in separate rings of kSlots slots each
  static constexpr int kFit = TV_ATTN_LDS_BUDGET / (2 * kTileBytes);
  static constexpr int kSlots = kFit < 2 ? 2 : (kFit > 4 ? 4 : kFit);
  static constexpr int kInstPerWave = kStageBytes / 1024 / kNW;  // 1 KB per wave DMA
  static constexpr int kDT = D / 16;  // 16-wide output column tiles
  // workgroups per CU the register budget is sized for: fp32 at D = 256 keeps
  // 64 query and 64 accumulator registers per lane and gets the whole file
  static constexpr int kMinWG =
      kTeams > 1 ? 1 : ((kEsz == 4 && D == 256) ? 1 : TV_ATTN_MIN_WG);
  static_assert(kInstPerWave >= 1 && kStageBytes % (1024 * kNW) == 0, "stage must split over waves");
  static_assert(kInstPerWave * (2 * kSlots - 1) <= 63, "vmcnt range");
};

// XOR key of a row's 16-byte granules: key(r) = 4 r0 ^ 8 r1 ^ 15 r2 ^ 6 r3 over
// the bits of r mod 16 (a bijection).  Chosen by timing every invertible
// linear key on gfx950: with it the K operand reads (16 rows, one granule each,
// ds_read_b128), the V transpose reads (4 rows, two adjacent granules each, per
// 16 lanes) and the fp32 V reads all run without bank conflicts, where the
// key r0..r3 -> r1 r2 r3 r0 made every K read a two-way conflict.
template <typename T, int D>
__device__ __forceinline__ int swz_key(int row) {
  using C = Cfg<T, D>;
  const int k = ((row & 3) << 2) ^ ((row & 4) ? 15 : 0) ^ ((row & 8) ? 6 : 0);
  return k & C::kSwz;
}

// Byte offset of (row, byte) in a tile slot under that swizzle.
template <typename T, int D>
__device__ __forceinline__ int swz(int row, int byte) {
  using C = Cfg<T, D>;
  return row * C::kRowBytes + (((byte >> 4) ^ swz_key<T, D>(row)) << 4) + (byte & 15);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (LDS DMA; the LDS base goes in M0 and must be wave-uniform).  Issued through
// asm so that the compiler's wait insertion does not drain the whole ring
// before each LDS read; completion is tracked with explicit vmcnt waits.
// kNT marks the load non-temporal: a stream read once streams faster past
// the caches (7.1 TB/s against 6.2 TB/s for a plain LDS DMA ring on MI355X).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool kNT = true>
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
  const uint32_t la = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(lds)));
  if constexpr (kNT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 ::"s"(la), "v"(src) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 ::"s"(la), "v"(src) : "memory", "m0");
}

#pragma clang diagnostic pop

// LDS transpose read of four bf16: within each 16-lane group, lane i receives
// element (i & 3) of the 8-byte rows addressed by lanes 4j + (i >> 2), j = 0..3.
__device__ __forceinline__ s16x4_t lds_read_tr16(const unsigned char* p) {
  auto lp = (__attribute__((address_space(3))) bf16x4_t*)(p);
  return __builtin_bit_cast(s16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// 32-bit LDS address of a shared array, and reads at such an address
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)(p)));
}
__device__ __forceinline__ u32x4_t lds_u4(uint32_t a) {
  return *(__attribute__((address_space(3))) const u32x4_t*)(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ s16x4_t lds_tr16(uint32_t a) {
  auto lp = (__attribute__((address_space(3))) bf16x4_t*)(static_cast<uintptr_t>(a));
  return __builtin_bit_cast(s16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that does not drain outstanding global loads (the
// __syncthreads fence would wait for every in-flight stage); LDS reads issued
// before it have completed.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until at most n vector-memory instructions issued later are in flight
// (n above 31 waits for 31, which is only stricter)
template <int M = 0>
__device__ __forceinline__ void wait_vm_upto(int n) {
  if constexpr (M < 31) {
    if (n == M) {
      wait_vmem<M>();
      return;
    }
    wait_vm_upto<M + 1>(n);
  } else {
    wait_vmem<31>();
  }
}

struct SeqPlan {
  int start, end, split_len, nsplit;
};

// Key range of one sequence and its split: with a window only keys at or after
// (smallest node position) + 1 - window can be visible.  The split length
// grows past the nominal one if the range needs more splits than were planned.
__device__ __forceinline__ SeqPlan seq_plan(int ctx_raw, int max_ctx, int window, int min_pos,
                                            int nsplit_max, int split_tokens) {
  SeqPlan p;
  const int ctx = min(max(ctx_raw, 0), max_ctx);
  int start = 0;
  if (window > 0) start = min(max(min_pos + 1 - window, 0), ctx);
  const int len = ctx - start;
  int sl = split_tokens;
  int need = (len + sl - 1) / sl;
  if (need > nsplit_max) {
    sl = ((len + nsplit_max - 1) / nsplit_max + kTile - 1) / kTile * kTile;
    need = (len + sl - 1) / sl;
  }
  p.start = start;
  p.end = ctx;
  p.split_len = sl;
  p.nsplit = max(need, 1);
  return p;
}

// smallest and largest position id of the tree (read by wave 0, lane l taking
// nodes l, l + 64, ...)
__device__ __forceinline__ int2 tree_pos_range(const int32_t* pos_b, int N, int2* s_rng) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    int lo = 0x7fffffff, hi = -0x7fffffff;
    // unconditional loads (node N - 1 past the tree), then selects: under a
    // condition each load would be waited for in its own branch
    int pv[TV_MAX_NODES / 64];
#pragma unroll
    for (int j = 0; j < TV_MAX_NODES / 64; ++j) pv[j] = pos_b[max(min(tid + 64 * j, N - 1), 0)];
#pragma unroll
    for (int j = 0; j < TV_MAX_NODES / 64; ++j) {
      const int i = tid + 64 * j;
      lo = i < N ? min(lo, pv[j]) : lo;
      hi = i < N ? max(hi, pv[j]) : hi;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off, 64));
      hi = max(hi, __shfl_xor(hi, off, 64));
    }
    if (tid == 0) *s_rng = make_int2(lo, hi);
  }
  __syncthreads();
  // the same value in every lane: make it wave-uniform, so that what is
  // derived from it (the split's key range, stage bounds) stays scalar
  const int2 r = *s_rng;
  return make_int2(__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// an empty asm that takes v in and out of a register: v is computed before
// this point and not moved past it
template <typename V>
__device__ __forceinline__ void pin(V& v) {
  asm volatile("" : "+v"(v));
}

// x = keep ? x : other, rewriting x's own register, so that a value that
// passes a branch masked on one side and untouched on the other needs no copy
// where the sides join
__device__ __forceinline__ float keep_or(float x, bool keep, float other) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
  asm volatile("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(x) : "v"(other), "s"(m));
  return x;
}

// The values of lanes l and l ^ S (S = 16 or 32), through the gfx950 lane-swap
// instructions (VALU, no LDS round trip): the two results hold exactly that
// pair, in an order that depends on the lane, so max and sum over them are the
// same in both lanes of the pair.
template <int S>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    static_assert(S == 32, "lane pairs are 16 or 32 apart");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}
template <int S>
__device__ __forceinline__ float pair_max(float v) {
  float a, b;
  lane_pair<S>(v, a, b);
  return fmaxf(a, b);
}
template <int S>
__device__ __forceinline__ float pair_sum(float v) {
  float a, b;
  lane_pair<S>(v, a, b);
  return a + b;
}

// Ancestor word that holds the node keys from key_base on (key_base a multiple
// of 32, so a tile's keys share it); selected, not indexed, so that the words
// stay in registers.
__device__ __forceinline__ uint64_t anc_word(const uint64_t (&a)[kAncW], int key_base) {
  uint64_t r = a[0];
#pragma unroll
  for (int w = 1; w < kAncW; ++w) r = (key_base >> 6) == w ? a[w] : r;
  return r;
}

// Query fragments (MFMA B operand: row lr, 8 (bf16) or 1 (fp32) dims per k
// step), position and ancestor words of one query row.  Loaded ahead of the
// plan and the page indices, so that these loads overlap theirs.
template <typename T, int D>
struct RowIn {
  static constexpr int kQ = (sizeof(T) == 2) ? D / 32 : D / 4;
  bf16x8_t qb[sizeof(T) == 2 ? kQ : 1];
  float qf[sizeof(T) == 4 ? kQ : 1];
  int pos;
  uint64_t anc[kAncW];  // words past the tree's word count are 0
};

// this lane's query row of row group rg of unit (b, g): R = rg * kRows + 16 *
// (wave within its team) + lr, node R / G, query head g * G + R % G
template <typename T, int D>
__device__ __forceinline__ RowIn<T, D> row_in(const T* __restrict__ q,
                                              const int32_t* __restrict__ pos_b,
                                              const uint64_t* __restrict__ anc, int b, int g,
                                              int rg, int N, int Hq, int G, int rows) {
  RowIn<T, D> ri;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int R = rg * kRows + (wave % kWaves) * 16 + lr;
  const bool row_ok = R < rows;
  const int t = row_ok ? R / G : 0;
  const int hl = row_ok ? R % G : 0;
  const size_t qoff = ((static_cast<size_t>(b) * N + t) * Hq + g * G + hl) * D;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < RowIn<T, D>::kQ; ++ks) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(q + qoff + ks * 32 + lg * 8)
                       : make_uint4(0, 0, 0, 0);
      ri.qb[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < RowIn<T, D>::kQ; ++ks) ri.qf[ks] = row_ok ? q[qoff + ks * 4 + lg] : 0.0f;
  }
  ri.pos = pos_b[t];
  const int nw = (N + 63) / 64;
#pragma unroll
  for (int w = 0; w < kAncW; ++w)
    ri.anc[w] = w < nw ? anc[(static_cast<size_t>(b) * N + t) * nw + w] : 0ull;
  return ri;
}

// page indices [p0, p0 + npages) of one sequence into s_pages (as far as it
// reaches), clamped into the pool; all loads go out before the first store.
// The loads are unconditional (lanes past the range read its last entry):
// under a condition the compiler waits for each load inside its branch, one
// memory round trip after another.
template <int NT, int kPages>
struct PageLoads {
  static constexpr int kPer = kPages / NT;
  static_assert(kPer * NT == kPages, "page cache layout");
  int n;
  int v[kPer];
};
template <int NT, int kPages>
__device__ __forceinline__ PageLoads<NT, kPages> pages_issue(const int32_t* __restrict__ bt_b, int p0, int npages) {
  PageLoads<NT, kPages> pl;
  pl.n = min(npages, kPages);
  // an empty range reads the row's first entry (p0 may lie past the row) and
  // stores nothing
  const int base = pl.n > 0 ? p0 : 0, last = max(pl.n - 1, 0);
#pragma unroll
  for (int k = 0; k < pl.kPer; ++k) pl.v[k] = bt_b[base + min(static_cast<int>(threadIdx.x) + k * NT, last)];
  return pl;
}
template <int NT, int kPages>
__device__ __forceinline__ void pages_store(int* s_pages, const PageLoads<NT, kPages>& pl, int num_blocks) {
#pragma unroll
  for (int k = 0; k < pl.kPer; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < pl.n) s_pages[i] = min(max(pl.v[k], 0), num_blocks - 1);
  }
}
template <int NT, int kPages>
__device__ __forceinline__ void fill_pages(int* s_pages, const int32_t* __restrict__ bt_b, int p0,
                                           int npages, int num_blocks) {
  pages_store<NT, kPages>(s_pages, pages_issue<NT, kPages>(bt_b, p0, npages), num_blocks);
}

// One segment of the key stream of one (sequence, kv head, row group): the
// context keys [k0, k1) and the node tiles [node_t0, node_t1) (32 nodes each),
// accumulated with an online softmax.  With final_out the normalised rows go
// to `out`; otherwise the unnormalised partial (acc, m, l) goes to partial
// slot `pslot`.  s_pos holds the tree's position ids and s_pages the page
// indices of pages k0 / 16 onwards, both filled by the caller before a
// barrier that this routine also relies on for its own LDS.
template <typename T, typename TO, int D, int kTeams, int kPages>
__device__ __forceinline__ void attn_segment(
    const RowIn<T, D>& ri, const T* __restrict__ kn, const T* __restrict__ vn,
    const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ bt_b,
    int num_blocks, const uint64_t* __restrict__ anc, const int32_t* __restrict__ pos_b, int N,
    int Hq, int Hkv, int G, int rows, int window, float scale_log2, int b, int g, int rg, int k0,
    int k1, int node_t0, int node_t1, int2 prng, bool final_out, size_t pslot,
    TO* __restrict__ out, float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
    unsigned char* kring, unsigned char* vring, const int* s_pages, const int* s_pos) {
  using C = Cfg<T, D, kTeams>;
  const int tid = threadIdx.x;
  // stages: context keys in stages of kStageKeys, then node stages [node_t0, node_t1)
  const int nctx_tiles = k1 > k0 ? (k1 - k0 + C::kStageKeys - 1) / C::kStageKeys : 0;
  const int ntiles = nctx_tiles + (node_t1 - node_t0);
  // context keys in [win_all, min_pos] are inside every row's window
  const int win_all = window > 0 ? prng.y - window + 1 : -0x7fffffff;
  const int p0 = k0 >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave / kWaves;  // which tile of each stage this wave computes
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int R = rg * kRows + (wave % kWaves) * 16 + lr;
  const bool row_ok = R < rows;
  const int t = row_ok ? R / G : 0;
  const int hl = row_ok ? R % G : 0;
  const size_t qoff = ((static_cast<size_t>(b) * N + t) * Hq + g * G + hl) * D;
  constexpr int kQ = RowIn<T, D>::kQ;
  bf16x8_t qf_b[sizeof(T) == 2 ? kQ : 1];
  float qf_f[sizeof(T) == 4 ? kQ : 1];
#pragma unroll
  for (int ks = 0; ks < (sizeof(T) == 2 ? kQ : 1); ++ks) qf_b[ks] = ri.qb[ks];
#pragma unroll
  for (int ks = 0; ks < (sizeof(T) == 4 ? kQ : 1); ++ks) qf_f[ks] = ri.qf[ks];
  const int row_pos = ri.pos;
  uint64_t row_anc[kAncW];
#pragma unroll
  for (int w = 0; w < kAncW; ++w) row_anc[w] = ri.anc[w];
  // make the query and row loads complete here, so that the compiler's wait
  // bookkeeping does not place a full drain inside the key loop
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) asm volatile("" ::"v"(qf_b[ks]));
  } else {
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) asm volatile("" ::"v"(qf_f[ks]));
  }
  asm volatile("" ::"v"(row_pos));
#pragma unroll
  for (int w = 0; w < kAncW; ++w) asm volatile("" ::"v"(row_anc[w]));

  f32x4_t acc[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  const unsigned char* kcb = reinterpret_cast<const unsigned char*>(kc);
  const unsigned char* vcb = reinterpret_cast<const unsigned char*>(vc);
  const unsigned char* knb = reinterpret_cast<const unsigned char*>(kn);
  const unsigned char* vnb = reinterpret_cast<const unsigned char*>(vn);
  // every earlier global access (query, row data, an earlier segment's stores)
  // completes here, so the counted waits below see only this segment's loads
  wait_vmem<0>();
  __syncthreads();  // page cache ready
  if (ntiles == 0) return;

  // Enqueue the loads of one tile's keys (or values) straight into its LDS
  // slot.  Each wave fills kInstPerWave 1 KB blocks; lane i of a block lands
  // at block + 16 i, so the lane picks the global granule that belongs there
  // under the swizzle.  Keys past the end of the range read a valid key
  // instead (masked later), so that LDS never holds non-finite garbage.
  auto issue = [&](int it, bool values) {
    unsigned char* dst = (values ? vring : kring) + (it % C::kSlots) * C::kStageBytes;
    const bool is_node = it >= nctx_tiles;
    const int base = is_node ? (node_t0 + it - nctx_tiles) * C::kStageKeys : k0 + it * C::kStageKeys;
    const int lim = is_node ? N : k1;
    const unsigned char* src = is_node ? (values ? vnb : knb) : (values ? vcb : kcb);
#pragma unroll
    for (int j = 0; j < C::kInstPerWave; ++j) {
      const int blk = wave * C::kInstPerWave + j;
      const int gl = blk * 64 + lane;
      const int row = gl / C::kGran;
      const int gp = gl % C::kGran;
      const int part = gp ^ swz_key<T, D>(row);
      const int key = min(base + row, lim - 1);
      size_t off;
      if (is_node) {
        off = ((static_cast<size_t>(b) * N + key) * Hkv + g) * C::kRowBytes;
      } else {
        const int pi = (key >> 4) - p0;
        const int page = pi < kPages ? s_pages[pi] : min(max(bt_b[key >> 4], 0), num_blocks - 1);
        off = ((static_cast<size_t>(page) * Hkv + g) * 16 + (key & 15)) * C::kRowBytes;
      }
      lds_dma16(src + off + part * 16, dst + blk * 1024);
    }
    asm volatile("" ::: "memory");
  };

  // Loads go out in the order K(0) V(0) K(1) V(1) ...: the prologue fills
  // every slot; afterwards K(it + kSlots) goes out once every wave is done
  // with the keys of tile it (second barrier of iteration it) and
  // V(it + kSlots) once every wave is done with its values (first barrier of
  // iteration it + 1).  While one tile's keys or values are in use, the next
  // 2 kSlots - 1 groups are in flight; two barriers per tile.
  for (int i = 0; i < C::kSlots && i < ntiles; ++i) {
    issue(i, false);
    issue(i, true);
  }

  for (int it = 0; it < ntiles; ++it) {
    const int newest = min(it + C::kSlots - 1, ntiles - 1);  // newest tile whose keys are out
    // values issued so far reach tile newest (prologue) or newest - 1
    const int v_out = it == 0 ? newest : min(it + C::kSlots - 2, ntiles - 1);
    // loads issued after K(it): V(it .. v_out) and K(it + 1 .. newest)
    wait_vm_upto(C::kInstPerWave * ((v_out - it + 1) + (newest - it)));
    lds_barrier();  // keys of tile `it` have landed; every wave is done with tile it - 1
    if (it > 0 && it + C::kSlots - 1 < ntiles) issue(it + C::kSlots - 1, true);

    const unsigned char* Kt = kring + (it % C::kSlots) * C::kStageBytes + team * C::kTileBytes;
    const unsigned char* Vt = vring + (it % C::kSlots) * C::kStageBytes + team * C::kTileBytes;
    const bool is_node = it >= nctx_tiles;
    const int base = (is_node ? (node_t0 + it - nctx_tiles) * C::kStageKeys : k0 + it * C::kStageKeys) +
                     team * kTile;
    const int lim = is_node ? N : k1;

    // S^T for two 16-key halves: lane holds keys 16j + 4lg + i of row lr
    f32x4_t S[2];
    if constexpr (sizeof(T) == 2) {
      // the two halves' products interleave (independent accumulators); key
      // fragments are read two k-steps ahead, and scheduling fences keep the
      // compiler from sinking the reads next to their use
      S[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      S[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      constexpr int kAh = kQ < 2 ? kQ : 2;
      uint4 ka[kAh + 1][2];
      auto kread = [&](int ks, int j) __attribute__((always_inline)) {
        return *reinterpret_cast<const uint4*>(Kt + swz<T, D>(16 * j + lr, ks * 64 + lg * 16));
      };
#pragma unroll
      for (int ks = 0; ks < kAh; ++ks) {
        ka[ks][0] = kread(ks, 0);
        ka[ks][1] = kread(ks, 1);
      }
#pragma unroll
      for (int ks = 0; ks < kQ; ++ks) {
        if (ks + kAh < kQ) {
          ka[(ks + kAh) % (kAh + 1)][0] = kread(ks + kAh, 0);
          ka[(ks + kAh) % (kAh + 1)][1] = kread(ks + kAh, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        S[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, ka[ks % (kAh + 1)][0]), qf_b[ks], S[0], 0, 0, 0);
        S[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, ka[ks % (kAh + 1)][1]), qf_b[ks], S[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int krow = 16 * j + lr;
      {
#pragma unroll
        for (int ks = 0; ks < kQ; ++ks) {
          float a = *reinterpret_cast<const float*>(Kt + swz<T, D>(krow, (ks * 4 + lg) * 4));
          S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf_f[ks], S[j], 0, 0, 0);
        }
      }
    }
    }

    // scale into the log2 domain and mask; a context tile that lies wholly
    // inside the range and inside every row's window needs no mask
    float x[2][4];
    const bool full = !is_node && base + kTile <= lim &&
                      (window <= 0 || (base >= win_all && base + kTile - 1 <= prng.x));
    if (full) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[j][i] = S[j][i] * scale_log2;
    } else {
      // a node tile's 32 keys share one ancestor word
      const uint64_t aw = anc_word(row_anc, base);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = base + 16 * j + 4 * lg + i;
          const int kpos = is_node ? s_pos[key & (TV_MAX_NODES - 1)] : key;
          const int dpos = row_pos - kpos;
          bool vis = row_ok & (key < lim);
          vis &= !is_node | (((aw >> (key & 63)) & 1ull) != 0ull);
          vis &= (window <= 0) | ((dpos >= 0) & (dpos < window));
          x[j][i] = vis ? S[j][i] * scale_log2 : -INFINITY;
        }
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    mt = pair_max<32>(pair_max<16>(mt));
    const float m_new = fmaxf(m_run, mt);
    // reference point for the exponentials (0 while the row has seen nothing)
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    float p[2][4];
    float ps = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[j][i] = fast_exp2(x[j][i] - m_use);
        ps += p[j][i];
      }
    // rescale only when some row's running max moved
    if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0ull) {
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) acc[dt] *= alpha;
    }
    l_run += ps;
    m_run = m_new;

    // loads issued after V(it): K and V of it + 1 .. newest
    wait_vm_upto(C::kInstPerWave * 2 * (newest - it));
    lds_barrier();  // values of tile `it` have landed; every wave is done with its keys
    if (it + C::kSlots < ntiles) issue(it + C::kSlots, false);

    // O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
      // P = P_hi + P_lo, both bf16: the two products keep P to ~16 mantissa
      // bits, so the bf16 MFMA adds no visible error to the weights
      bf16x8_t ph, pl;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 h = static_cast<__bf16>(p[j][i]);
          ph[4 * j + i] = h;
          pl[4 * j + i] = static_cast<__bf16>(p[j][i] - static_cast<float>(h));
        }
      // lane (lr, lg) addresses value row 4lg + (lr >> 2) (and 16 + that),
      // columns 16 dt + 4 (lr & 3) .. +3; the transpose read hands lane lr
      // column 16 dt + lr of rows 4lg + 0..3 (and 16 + 4lg + 0..3)
      const int vrow = 4 * lg + (lr >> 2);
      const int vcol = 8 * (lr & 3);
      // value reads run two column tiles ahead of the products (fenced as above)
      constexpr int kVA = C::kDT < 2 ? C::kDT : 2;
      s16x4_t vlo[kVA + 1], vhi[kVA + 1];
#pragma unroll
      for (int dt = 0; dt < kVA; ++dt) {
        vlo[dt] = lds_read_tr16(Vt + swz<T, D>(vrow, dt * 32 + vcol));
        vhi[dt] = lds_read_tr16(Vt + swz<T, D>(16 + vrow, dt * 32 + vcol));
      }
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
        if (dt + kVA < C::kDT) {
          vlo[(dt + kVA) % (kVA + 1)] = lds_read_tr16(Vt + swz<T, D>(vrow, (dt + kVA) * 32 + vcol));
          vhi[(dt + kVA) % (kVA + 1)] =
              lds_read_tr16(Vt + swz<T, D>(16 + vrow, (dt + kVA) * 32 + vcol));
        }
        __builtin_amdgcn_sched_barrier(0);
        const s16x4_t lo = vlo[dt % (kVA + 1)];
        const s16x4_t hi = vhi[dt % (kVA + 1)];
        const s16x8_t av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl, acc[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int krow = 16 * j + 4 * lg + i;
#pragma unroll
          for (int dt = 0; dt < C::kDT; ++dt)
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                *reinterpret_cast<const float*>(Vt + swz<T, D>(krow, (dt * 16 + lr) * 4)), p[j][i],
                acc[dt], 0, 0, 0);
        }
    }
  }

  // row sum over the four lanes that share the row
  float l_tot = pair_sum<32>(pair_sum<16>(l_run));
  if constexpr (kTeams > 1) {
    // teams above the first hand (m, l, acc) of their rows to the first team
    // through LDS (the rings are free now); the first team merges them
    static_assert(kTeams == 2, "two teams");
    static_assert(kWaves * C::kDT * 64 * 16 <= C::kSlots * C::kStageBytes, "merge fits");
    __syncthreads();  // every wave is done with the rings
    float* mb_acc = reinterpret_cast<float*>(kring);   // [wave][dt][lane][4]
    float2* mb_ml = reinterpret_cast<float2*>(vring);  // [wave][lane] (m, l)
    const int wt = wave % kWaves;
    if (team == 1) {
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt)
        *reinterpret_cast<f32x4_t*>(mb_acc + ((wt * C::kDT + dt) * 64 + lane) * 4) = acc[dt];
      mb_ml[wt * 64 + lane] = make_float2(m_run, l_tot);
    }
    __syncthreads();
    if (team == 1) return;
    const float2 o = mb_ml[wt * 64 + lane];
    const float m_new = fmaxf(m_run, o.x);  // finite: every row sees its own node
    const float c0 = fast_exp2(m_run - m_new), c1 = fast_exp2(o.x - m_new);
    // explicit fmaf: both output types' instantiations round alike
    l_tot = __builtin_fmaf(o.y, c1, l_tot * c0);
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      const f32x4_t t1 = *reinterpret_cast<const f32x4_t*>(mb_acc + ((wt * C::kDT + dt) * 64 + lane) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[dt][r] = __builtin_fmaf(t1[r], c1, acc[dt][r] * c0);
    }
    m_run = m_new;
  }
  if (!row_ok) return;

  if (final_out) {
    const float inv = 1.0f / l_tot;
    TO* o = out + qoff;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      const int d0 = dt * 16 + 4 * lg;
      if constexpr (sizeof(TO) == 2) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(acc[dt][0] * inv)) |
              (static_cast<uint32_t>(f32_to_bf16(acc[dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(acc[dt][2] * inv)) |
              (static_cast<uint32_t>(f32_to_bf16(acc[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(o + d0) = w;
      } else {
        *reinterpret_cast<float4*>(o + d0) =
            make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
      }
    }
  } else {
    const size_t ub = pslot * rows + R;
    float* pa = ws_acc + ub * D;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt)
      *reinterpret_cast<float4*>(pa + dt * 16 + 4 * lg) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (lg == 0) ws_ml[ub] = make_float2(m_run, l_tot);
  }
}


// Teams per workgroup of the per-unit layout: two, when two stages of both
// rings fit in 128 KB of LDS (one such workgroup per CU).
template <typename T, int D>
constexpr int split_teams() {
  return 2 * 2 * 2 * kTile * D * static_cast<int>(sizeof(T)) <= 131072 ? 2 : 1;
}

template <typename T, typename TO, int D>
__global__ __launch_bounds__((kThreads * split_teams<T, D>()), 1) void attn_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kn, const T* __restrict__ vn,
    const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ bt,
    int max_blocks, int num_blocks, const int32_t* __restrict__ ctx_len, int max_ctx,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ pos, int N, int Hq, int Hkv,
    int G, int rows, int row_groups, int nsplit_max, int split_tokens, int window,
    float scale_log2, int units, TO* __restrict__ out, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml) {
  constexpr int kSplitTeams = split_teams<T, D>();
  using C = Cfg<T, D, kSplitTeams>;
  __shared__ __align__(1024) unsigned char kring[C::kSlots * C::kStageBytes];
  __shared__ __align__(1024) unsigned char vring[C::kSlots * C::kStageBytes];
  __shared__ int s_pages[kSplitPages];
  __shared__ int s_pos[TV_MAX_NODES];
  __shared__ int2 s_rng;

  // Blocks are dealt round-robin to the 8 XCDs.  Work units are numbered
  // split-major, u = s * (B * Hkv) + b * Hkv + g, and consecutive units go to
  // different XCDs, so each XCD gets the same share of every sequence (with 8
  // kv heads, one head of each): a ragged batch loads the XCDs evenly.  The
  // row groups of one unit, which stream the same keys, share an XCD and its L2.
  const int xcd = blockIdx.x % 8;
  const int slot = blockIdx.x / 8;
  const int u = (slot / row_groups) * 8 + xcd;
  if (u >= units) return;
  const int rg = slot % row_groups;
  const int n_bg = units / nsplit_max;  // B * Hkv
  const int s = u / n_bg;
  const int g = (u % n_bg) % Hkv;
  const int b = (u % n_bg) / Hkv;

  const int tid = threadIdx.x;
  const int32_t* pos_b = pos + static_cast<size_t>(b) * N;
  // the context length and this lane's query row go out with the tree positions
  const int ctx_raw = ctx_len[b];
  const RowIn<T, D> ri = row_in<T, D>(q, pos_b, anc, b, g, rg, N, Hq, G, rows);
  if (tid < TV_MAX_NODES) s_pos[tid] = tid < N ? pos_b[tid] : 0;
  const int2 prng = tree_pos_range(pos_b, N, &s_rng);
  const SeqPlan sp = seq_plan(ctx_raw, max_ctx, window, prng.x, nsplit_max, split_tokens);
  if (s >= sp.nsplit) return;  // uniform over the workgroup
  const int k0 = sp.start + s * sp.split_len;
  const int k1 = min(k0 + sp.split_len, sp.end);
  const bool last = s == sp.nsplit - 1;

  // page indices of this split, clamped into the pool
  const int32_t* bt_b = bt + static_cast<size_t>(b) * max_blocks;
  const int p0 = k0 >> 4;
  const int npages = k1 > k0 ? ((k1 - 1) >> 4) - p0 + 1 : 0;
  fill_pages<kThreads * kSplitTeams, kSplitPages>(s_pages, bt_b, p0, npages, num_blocks);

  attn_segment<T, TO, D, kSplitTeams, kSplitPages>(ri, kn, vn, kc, vc, bt_b, num_blocks, anc, pos_b, N, Hq, Hkv, G,
                         rows, window, scale_log2, b, g, rg, k0, k1, 0,
                         last ? (N + C::kStageKeys - 1) / C::kStageKeys : 0,
                         prng, sp.nsplit == 1,
                         (static_cast<size_t>(b) * Hkv + g) * nsplit_max + s, out, ws_acc, ws_ml,
                         kring, vring, s_pages, s_pos);
}

// Online softmax of one row tile over a tile's masked, log2-scaled scores x
// (as in attn_segment): running max and sum, rescaling the accumulator when
// some row's max moved; p receives the tile's weights.
template <int kDT>
__device__ __forceinline__ void tile_softmax_w(const float x[2][4], float& m_run, float& l_run,
                                               f32x4_t* acc, float p[2][4]) {
  float mt = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                   fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
  mt = pair_max<32>(pair_max<16>(mt));
  const float m_new = fmaxf(m_run, mt);
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  float ps = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[j][i] = fast_exp2(x[j][i] - m_use);
      ps += p[j][i];
    }
  if (__builtin_amdgcn_ballot_w64(m_new != m_run) != 0ull) {
    const float alpha = fast_exp2(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) acc[dt] *= alpha;
  }
  l_run += ps;
  m_run = m_new;
}

// a finished row: the normalised output, or the partial (acc, m, l) in row ub
template <typename TO, int D>
__device__ __forceinline__ void wide_row_store(bool final_out, const f32x4_t* acc, float m_run,
                                               float l_tot, int lg, TO* __restrict__ o,
                                               float* __restrict__ ws_acc,
                                               float2* __restrict__ ws_ml, size_t ub) {
  constexpr int kDT = D / 16;
  if (final_out) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const int d0 = dt * 16 + 4 * lg;
      if constexpr (sizeof(TO) == 2) {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16(acc[dt][0] * inv)) |
              (static_cast<uint32_t>(f32_to_bf16(acc[dt][1] * inv)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16(acc[dt][2] * inv)) |
              (static_cast<uint32_t>(f32_to_bf16(acc[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(o + d0) = w;
      } else {
        *reinterpret_cast<float4*>(o + d0) =
            make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
      }
    }
  } else {
    float* pa = ws_acc + ub * D;
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *reinterpret_cast<float4*>(pa + dt * 16 + 4 * lg) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (lg == 0) ws_ml[ub] = make_float2(m_run, l_tot);
  }
}

// Query tiles wider than one workgroup of 64 rows (G * N > 64, for instance
// 8 query heads per kv head times 64 nodes = 512 rows).  Each wave carries
// kRT tiles of 16 rows, so a workgroup covers 16 kRT * 8 rows of a unit and
// each key or value fragment read from LDS feeds kRT products; the row
// groups of a unit no longer stream the same keys once per 64 rows.  Keys
// go through the ring in stages of two 32-key tiles (one at D = 256), and
// the softmax runs once per stage.  Same work units (unit, row group, split),
// masking and partials as the per-unit layout; bf16 inputs.
//
// This layout is bound by the matrix and vector units, which on gfx950 issue
// to one SIMD nearly one after the other: every vector instruction adds to
// the stage time.  P therefore enters P.V as one bf16 product (the per-unit
// layout, bound by HBM, also carries P's rounding residual), and the softmax
// sums come from the matrix unit: P times a tile of ones, accumulated and
// rescaled like the output, so each row is normalised by the sum of exactly
// the bf16 weights its output was formed with.  The softmax reference
// follows each row's running maximum exactly, so a row's largest weight is
// 1 and rounds without error: rows dominated by a few keys, whose outputs
// stand far above the batch's RMS, keep their error small.  Against exact
// arithmetic the output then differs by the relative rounding of the other
// weights (2^-9), which averages out over the keys: under 1% of the output's
// RMS on N(0, 1) inputs.
//
// All eight waves (two per SIMD) run one software pipeline.  Iteration i
// forms the scores of stage i, then runs the P.V products of stage i - 1
// with the softmax of stage i spread between them, a few work items per
// product step: a wave issues vector instructions only every few cycles, so
// the softmax is hidden in the gaps of its own matrix stream rather than in
// another wave's (the two waves of a SIMD keep the matrix unit fed between
// them).  P.V walks the key tiles in order, so the bf16 probabilities of
// stage i's first key tile overwrite stage i - 1's once its products are
// done and the last key tile's follow the products: one probability buffer.
// A move of a row's softmax reference rescales the accumulators after that
// stage's products.  One barrier per stage: behind it the keys of stage i
// and the values of stage i - 1 have landed, and every wave is done with
// the keys of stage i - 1 and the values of stage i - 2, whose slots each
// wave refills with its share of the loads.  These loads keep the default
// cache policy: the row groups of a unit read the same keys through L2.
template <int D>
constexpr int wide_tiles() {
  return D == 256 ? 1 : 2;
}
constexpr int kWideWaves = 8;

template <typename TO, int D>
__global__ __launch_bounds__(64 * kWideWaves, 1) void attn_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kn,
    const uint16_t* __restrict__ vn, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ bt, int max_blocks,
    int num_blocks, const int32_t* __restrict__ ctx_len, int max_ctx,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ pos, int N, int Hq, int Hkv,
    int G, int rows, int row_groups, int nsplit_max, int split_tokens, int window,
    float scale_log2, int units, TO* __restrict__ out, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml) {
  using T = uint16_t;
  using C = Cfg<T, D>;
  constexpr int kRT = wide_tiles<D>();
  constexpr int kW = kWideWaves;
  constexpr int kNT = 64 * kW;
  constexpr int kKT = D == 256 ? 1 : 2;                  // 32-key tiles per stage
  constexpr int kSK = kKT * kTile;                       // keys per stage
  constexpr int kSB = kKT * C::kTileBytes;               // bytes of a stage (keys or values)
  constexpr int kFitW = 131072 / (2 * kSB);
  constexpr int kSlots = kFitW > 6 ? 6 : kFitW;
  // every wave issues kIPW 1 KB loads per stage (keys or values)
  constexpr int kIPW = kSB / 1024 / kW;
  static_assert(kSlots >= 3, "the ring holds the keys of stage i + 1 while stage i is in use");
  static_assert(kIPW >= 1 && kIPW * 1024 * kW == kSB, "stage must split over the waves");
  static_assert(kIPW * (2 * kSlots - 1) <= 63, "vmcnt range");
  constexpr int kQ = D / 32;  // k steps of the score products
  __shared__ __align__(1024) unsigned char kring[kSlots * kSB];
  __shared__ __align__(1024) unsigned char vring[kSlots * kSB];
  __shared__ int s_pages[kSplitPages];
  __shared__ int s_pos[TV_MAX_NODES];
  __shared__ uint64_t s_anc[TV_MAX_NODES][kAncW];
  __shared__ int2 s_rng;

  // work units as in the per-unit layout: split-major, XCD-interleaved, the
  // row groups of one unit on one XCD
  const int xcd = blockIdx.x % 8;
  const int slot = blockIdx.x / 8;
  const int u = (slot / row_groups) * 8 + xcd;
  if (u >= units) return;
  const int rg = slot % row_groups;
  const int n_bg = units / nsplit_max;  // B * Hkv
  const int s = u / n_bg;
  const int g = (u % n_bg) % Hkv;
  const int b = (u % n_bg) / Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int32_t* pos_b = pos + static_cast<size_t>(b) * N;

  // rows R = (rg kW + wave) 16 kRT + 16 rt + lr (node R / G); their queries
  // go out with the context length, the tree's positions and ancestor words
  // to LDS (read only by masked stages)
  const int ctx_raw = ctx_len[b];
  int Rr[kRT], tn[kRT];
  bool ok[kRT];
  bf16x8_t qf[kRT][kQ];
  const int nw = (N + 63) / 64;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    Rr[rt] = (rg * kW + wave) * 16 * kRT + 16 * rt + lr;
    ok[rt] = Rr[rt] < rows;
    tn[rt] = ok[rt] ? Rr[rt] / G : 0;
    const int hl = ok[rt] ? Rr[rt] % G : 0;
    const size_t qoff = ((static_cast<size_t>(b) * N + tn[rt]) * Hq + g * G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) {
      const uint4 v = ok[rt] ? *reinterpret_cast<const uint4*>(q + qoff + ks * 32 + lg * 8)
                             : make_uint4(0, 0, 0, 0);
      qf[rt][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  if (tid < TV_MAX_NODES) s_pos[tid] = tid < N ? pos_b[tid] : 0;
  for (int i = tid; i < TV_MAX_NODES * kAncW; i += kNT) {
    const int t = i / kAncW, w = i % kAncW;
    s_anc[t][w] = (t < N && w < nw) ? anc[(static_cast<size_t>(b) * N + t) * nw + w] : 0ull;
  }
  const int2 prng = tree_pos_range(pos_b, N, &s_rng);
  const SeqPlan sp = seq_plan(ctx_raw, max_ctx, window, prng.x, nsplit_max, split_tokens);
  if (s >= sp.nsplit) return;  // uniform over the workgroup
  const int k0 = sp.start + s * sp.split_len;
  const int k1 = min(k0 + sp.split_len, sp.end);
  const bool last = s == sp.nsplit - 1;
  const bool final_out = sp.nsplit == 1;
  const size_t pslot = (static_cast<size_t>(b) * Hkv + g) * nsplit_max + s;
  const int32_t* bt_b = bt + static_cast<size_t>(b) * max_blocks;
  const int p0 = k0 >> 4;
  const int npages = k1 > k0 ? ((k1 - 1) >> 4) - p0 + 1 : 0;
  fill_pages<kNT, kSplitPages>(s_pages, bt_b, p0, npages, num_blocks);

  // make the row loads complete here (see attn_segment)
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) asm volatile("" ::"v"(qf[rt][ks]));
  }
  // acc: O^T column tiles; acc_l: the product of P with a tile of ones, whose
  // every element is the row's softmax sum over the same bf16 probabilities
  f32x4_t acc[kRT][C::kDT], acc_l[kRT];
  float m_run[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) acc[rt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc_l[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[rt] = -INFINITY;
  }
  // stages: context keys [k0, k1) in stages of kSK, then the node keys
  const int nctx = k1 > k0 ? (k1 - k0 + kSK - 1) / kSK : 0;
  const int ntiles = nctx + (last ? (N + kSK - 1) / kSK : 0);
  const int win_all = window > 0 ? prng.y - window + 1 : -0x7fffffff;
  const unsigned char* kcb = reinterpret_cast<const unsigned char*>(kc);
  const unsigned char* vcb = reinterpret_cast<const unsigned char*>(vc);
  const unsigned char* knb = reinterpret_cast<const unsigned char*>(kn);
  const unsigned char* vnb = reinterpret_cast<const unsigned char*>(vn);
  wait_vmem<0>();
  __syncthreads();  // page cache ready

  // Loads of stage keys (or values) into their slot: stage row r is row r % 32
  // of tile r / 32, swizzled as in the per-unit layout.  Load j of a wave
  // fills the 1 KB block wave kIPW + j of the slot: its lane takes granule
  // (gl % kGran) ^ key of stage row gl / kGran, gl = (wave kIPW + j) 64 + lane.
  // Lane coordinates are formed where they are used, from a copy of the lane
  // index the compiler cannot see through, so that no part of the address
  // arithmetic is hoisted into registers held across the stream.
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto ld_row = [&](int j, int l) __attribute__((always_inline)) {
    return ((wave * kIPW + j) * 64 + l) / C::kGran;
  };
  auto ld_gran = [&](int j, int l) __attribute__((always_inline)) {
    const int r = ld_row(j, l);
    return ((((wave * kIPW + j) * 64 + l) % C::kGran) ^ swz_key<T, D>(r));
  };
  // the loads of one half (values or keys) of stage st, issued at once, each
  // lane's page read from the cache (any stage: partial, windowed or nodes)
  auto issue_stage = [&](int st, bool values) __attribute__((always_inline)) {
    if (st >= ntiles) return;
    const bool is_node = st >= nctx;
    const int base = is_node ? (st - nctx) * kSK : k0 + st * kSK;
    const int lim = is_node ? N : k1;
    const unsigned char* src = is_node ? (values ? vnb : knb) : (values ? vcb : kcb);
    unsigned char* dst = (values ? vring : kring) + (st % kSlots) * kSB;
    const int l = opaque_lane();
    int key[kIPW], page[kIPW];
#pragma unroll
    for (int j = 0; j < kIPW; ++j) {
      key[j] = min(base + ld_row(j, l), lim - 1);
      page[j] = s_pages[min(max((key[j] >> 4) - p0, 0), kSplitPages - 1)];
    }
#pragma unroll
    for (int j = 0; j < kIPW; ++j) {
      const size_t off =
          is_node ? ((static_cast<size_t>(b) * N + key[j]) * Hkv + g) * C::kRowBytes
                  : ((static_cast<size_t>(page[j]) * Hkv + g) * 16 + (key[j] & 15)) * C::kRowBytes;
      lds_dma16<false>(src + off + ld_gran(j, l) * 16, dst + (wave * kIPW + j) * 1024);
    }
  };
  auto refill = [&](int sv, int sk) __attribute__((always_inline)) {
    issue_stage(sv, true);
    issue_stage(sk, false);
    asm volatile("" ::: "memory");
  };

  // The steady-state refills (values of stage sv, keys of stage sk), set up
  // right after the scores.  A context stage that lies wholly inside the
  // split and starts on a page boundary gives each wave rows of a single
  // page: its page base is one wave-uniform value and each load adds its
  // lane's offset inside the page.  When both halves are such stages their
  // loads are issued one by one between the products of P.V (load q is
  // value load q for q < kIPW, then key load q - kIPW), so that no issue
  // stalls on a full memory pipeline; otherwise they all go out at once.
  constexpr int kRowsW = kIPW * 64 / C::kGran;  // stage rows one wave fills
  static_assert(kRowsW <= 16 && 16 % kRowsW == 0, "a wave's rows share a page");
  const unsigned char* pre_base[2];  // per half: the page base (wave-uniform)
  int pre_dst[2];                    // LDS byte offset of the half's slot
  int page_off[kIPW];  // load j's byte offset inside a page (row and granule)
#pragma unroll
  for (int j = 0; j < kIPW; ++j) page_off[j] = (ld_row(j, lane) & 15) * C::kRowBytes + ld_gran(j, lane) * 16;
  auto issue_prepared = [&](int q) __attribute__((always_inline)) {
    const int half = q / kIPW, j = q % kIPW;
    const int off = page_off[j];
    unsigned char* dst = (half == 0 ? vring : kring) + pre_dst[half] + (wave * kIPW + j) * 1024;
    lds_dma16<false>(pre_base[half] + off, dst);
  };
  // The page of each half's rows, read from the page cache before the
  // scores' key reads fill the LDS queue (read after them, it waited behind
  // them); a stage past the split reads a clamped, unused entry.
  int pre_page[2];
  auto fetch_pages = [&](int sv, int sk) __attribute__((always_inline)) {
    const int st[2] = {sv, sk};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = ((k0 + st[q] * kSK + wave * kRowsW) >> 4) - p0;
      pre_page[q] = s_pages[min(max(idx, 0), kSplitPages - 1)];
    }
  };
  // returns whether the loads are left to P.V
  auto prepare = [&](int sv, int sk) __attribute__((always_inline)) {
    const int st[2] = {sv, sk};
    bool fast[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      pre_dst[q] = (st[q] % kSlots) * kSB;
      const bool is_node = st[q] >= nctx;
      const int base = is_node ? (st[q] - nctx) * kSK : k0 + st[q] * kSK;
      const int lim = is_node ? N : k1;
      fast[q] = st[q] < ntiles && !is_node && (base & 15) == 0 && base + kSK <= lim;
      pre_base[q] = kcb;
      if (fast[q]) {
        const int page = __builtin_amdgcn_readfirstlane(pre_page[q]);
        pre_base[q] = (q == 0 ? vcb : kcb) +
                      (static_cast<size_t>(page) * Hkv + g) * (16 * C::kRowBytes);
      }
    }
    if (fast[0] && fast[1]) return true;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (fast[q]) {
#pragma unroll
        for (int j = 0; j < kIPW; ++j) issue_prepared(q * kIPW + j);
      } else {
        issue_stage(st[q], q == 0);
      }
    }
    asm volatile("" ::: "memory");
    return false;
  };

  // Operand reads address the ring by 32-bit LDS offsets.  The swizzle XORs
  // only the granule bits of a row, and the slots are 1 KB aligned, so the
  // granule steps of a lane's reads are XORs on one lane base: k step ks adds
  // 4 ks to the granule (XOR ks << 6), column tile dt adds 2 dt (XOR dt << 5);
  // the second 16 rows and the second key tile are plain offsets.
  static_assert(4 * (kQ - 1) < C::kGran && 2 * (C::kDT - 1) < C::kGran, "steps stay in the row");
  const uint32_t kring_a = lds_addr(kring), vring_a = lds_addr(vring);
  const uint32_t k_lane = swz<T, D>(lr, lg * 16);
  const uint32_t v_lane = swz<T, D>(4 * lg + (lr >> 2), 8 * (lr & 3));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  f32x4_t S[kRT][2 * kKT];  // a stage's scores, masked, then its probabilities (in place)
  bf16x8_t ph[kRT][kKT];  // its probabilities in bf16

  // S^T of every row tile for the 16-key quarters of stage `it`: the key
  // fragments of a k step are read once (two k steps ahead) and feed all kRT
  // row tiles
  auto scores = [&](int it) __attribute__((always_inline)) {
    const uint32_t kb = kring_a + (it % kSlots) * kSB + k_lane;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int h = 0; h < 2 * kKT; ++h) S[rt][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
      constexpr int kAh = kQ < 2 ? kQ : 2;
      u32x4_t ka[kAh + 1][2];
      auto kread = [&](int ks, int j) __attribute__((always_inline)) {
        return lds_u4((kb ^ (ks << 6)) + j * 16 * C::kRowBytes + kt * C::kTileBytes);
      };
#pragma unroll
      for (int ks = 0; ks < kAh; ++ks) {
        ka[ks][0] = kread(ks, 0);
        ka[ks][1] = kread(ks, 1);
      }
#pragma unroll
      for (int ks = 0; ks < kQ; ++ks) {
        if (ks + kAh < kQ) {
          ka[(ks + kAh) % (kAh + 1)][0] = kread(ks + kAh, 0);
          ka[(ks + kAh) % (kAh + 1)][1] = kread(ks + kAh, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          S[rt][2 * kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ka[ks % (kAh + 1)][0]), qf[rt][ks], S[rt][2 * kt], 0, 0, 0);
          S[rt][2 * kt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ka[ks % (kAh + 1)][1]), qf[rt][ks], S[rt][2 * kt + 1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Softmax of stage `it` in the log2 domain, as work items that P.V spreads
  // over its steps.  Masks run only on partial stages, as one straight block
  // per kind of stage, before the products.  The scale is positive, so row
  // maxima are taken on the raw scores and the scale folds into one fma per
  // score.  The reference point m is the row's running maximum: weights are
  // at most 1, and a wave rescales its accumulators only on stages where
  // some row's maximum grew (a few percent of a long stream).  P goes to
  // bf16 pairs at a time (keys 16 h + 4 lg + i).
  float alpha[kRT], neg_m[kRT];
  bool need[kRT];
  auto mask_scores = [&](int it) __attribute__((always_inline)) {
    const bool is_node = it >= nctx;
    const int base = is_node ? (it - nctx) * kSK : k0 + it * kSK;
    const int lim = is_node ? N : k1;
    const bool full = !is_node && base + kSK <= lim &&
                      (window <= 0 || (base >= win_all && base + kSK - 1 <= prng.x));
    if (full) return;
    const float ninf = -INFINITY;
    if (is_node) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const int rpos = s_pos[tn[rt]];
        const uint64_t aw = s_anc[tn[rt]][(base >> 6) & (kAncW - 1)];  // a stage lies within one word
#pragma unroll
        for (int h = 0; h < 2 * kKT; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = base + 16 * h + 4 * lg + i;
            const int dpos = rpos - s_pos[key & (TV_MAX_NODES - 1)];
            bool vis = ok[rt] & (key < lim) & (((aw >> (key & 63)) & 1ull) != 0ull);
            vis &= (window <= 0) | ((dpos >= 0) & (dpos < window));
            S[rt][h][i] = keep_or(S[rt][h][i], vis, ninf);
          }
      }
    } else {
      // key = c + 4 lg with c = base + 16 h + i wave-uniform: only 4 lg and
      // the row's position minus 4 lg vary over the lanes
      const int l4 = 4 * lg;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const int pr = s_pos[tn[rt]] - l4;
#pragma unroll
        for (int h = 0; h < 2 * kKT; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = base + 16 * h + i;
            bool vis = ok[rt] & (l4 < lim - c);
            vis &= (window <= 0) | ((pr >= c) & (pr < c + window));
            S[rt][h][i] = keep_or(S[rt][h][i], vis, ninf);
          }
      }
    }
  };
  // Work items.  Phase 1: the kRT row maxima, then per key tile and row tile
  // the two exponential quarters of that tile.  Phase 2: the bf16 conversion
  // of key tile 0 (into the buffer P.V has finished with), and phase 3, after
  // the products, that of the last key tile.
  constexpr int kN1 = kRT + 2 * kKT * kRT;
  auto item_max = [&](int rt) __attribute__((always_inline)) {
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2 * kKT; ++h)
      mt = fmaxf(mt, fmaxf(fmaxf(S[rt][h][0], S[rt][h][1]), fmaxf(S[rt][h][2], S[rt][h][3])));
    mt = pair_max<32>(pair_max<16>(mt));
    const float mc = mt * scale_log2;
    need[rt] = mc > m_run[rt];
    // rows that keep their reference scale by exactly 1 (also rows still
    // at -inf, where the difference of references would be NaN)
    alpha[rt] = need[rt] ? fast_exp2(m_run[rt] - mc) : 1.0f;  // 0 from -inf
    m_run[rt] = need[rt] ? mc : m_run[rt];
    neg_m[rt] = m_run[rt] == -INFINITY ? 0.0f : -m_run[rt];
    pin(alpha[rt]);
    pin(neg_m[rt]);
  };
  auto item_exp = [&](int rt, int h) __attribute__((always_inline)) {
    f32x4_t e;
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = fast_exp2(fmaf(S[rt][h][i], scale_log2, neg_m[rt]));
    S[rt][h] = e;
    pin(S[rt][h]);
  };
  auto item_split = [&](int rt, int kt) __attribute__((always_inline)) {
    uint32_t hw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // fragment elements 2e, 2e + 1: quarter 2 kt + e / 2, keys 4 lg + 2 (e % 2) + 0, 1
      const f32x2_t f = {S[rt][2 * kt + e / 2][2 * (e % 2)], S[rt][2 * kt + e / 2][2 * (e % 2) + 1]};
      hw[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    }
    ph[rt][kt] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    pin(ph[rt][kt]);
  };
  // phase-1 item w (an item's results are pinned where it runs, so that the
  // compiler keeps the items between the product steps they were placed in)
  auto item1 = [&](int w) __attribute__((always_inline)) {
    if (w < kRT) {
      item_max(w);
    } else {
      const int kt = (w - kRT) / (2 * kRT), r = (w - kRT) % (2 * kRT);
      item_exp(r / 2, 2 * kt + r % 2);
    }
  };
  auto soft_all = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < kN1; ++w) item1(w);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) item_split(rt, kt);
  };
  // a row's reference moved: its accumulators and sum follow (after the
  // products of the previous stage)
  auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      if (__builtin_amdgcn_ballot_w64(need[rt]) != 0ull) {
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) acc[rt][dt] *= alpha[rt];
        acc_l[rt] *= alpha[rt];
      }
    }
  };

  // O^T += V^T P^T for stage `it`, key tile by key tile: the value fragments
  // of a column tile feed all row tiles; reads run two steps ahead.  With
  // `soft`, the softmax of the next stage runs in the gaps: phase 1 over the
  // first kS1 steps, phase 2 (key tile 0's conversion, once key tile 0 is done)
  // over the rest, phase 3 after the last step.
  constexpr int kSteps = C::kDT * kKT;  // (key tile, column tile) pairs
  constexpr int kS1 = kKT == 2 ? kSteps - C::kDT / 2 : kSteps;
  static_assert(kKT == 1 || kS1 >= C::kDT, "key tile 0 is done before its split");
  auto pv_product = [&](int it, bool with_loads, bool soft) __attribute__((always_inline)) {
    const uint32_t vb = vring_a + (it % kSlots) * kSB + v_lane;
    constexpr int kVA = 2;
    constexpr int kEvery = kSteps / (2 * kIPW);  // steps per prepared load
    static_assert(kEvery >= 1 && kEvery * 2 * kIPW == kSteps, "prepared loads spread over the steps");
    s16x4_t vlo[kVA + 1], vhi[kVA + 1];
    auto vread = [&](int st, s16x4_t& lo, s16x4_t& hi) __attribute__((always_inline)) {
      const int kt = st / C::kDT, dt = st % C::kDT;
      const uint32_t a = (vb ^ (dt << 5)) + kt * C::kTileBytes;
      lo = lds_tr16(a);
      hi = lds_tr16(a + 16 * C::kRowBytes);
    };
#pragma unroll
    for (int st = 0; st < kVA; ++st) vread(st, vlo[st], vhi[st]);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      if (st + kVA < kSteps) vread(st + kVA, vlo[(st + kVA) % (kVA + 1)], vhi[(st + kVA) % (kVA + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      const int kt = st / C::kDT, dt = st % C::kDT;
      const s16x4_t lo = vlo[st % (kVA + 1)];
      const s16x4_t hi = vhi[st % (kVA + 1)];
      const s16x8_t av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph[rt][kt], acc[rt][dt], 0, 0, 0);
        // the row sums, once per key tile
        if (dt == C::kDT - 1)
          acc_l[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, ph[rt][kt], acc_l[rt], 0, 0, 0);
      }
      if (with_loads && st % kEvery == kEvery - 1) issue_prepared(st / kEvery);
      if (soft) {
        if (st < kS1) {
#pragma unroll
          for (int w = st * kN1 / kS1; w < (st + 1) * kN1 / kS1; ++w) item1(w);
        } else if (kKT == 2) {
          constexpr int kS2 = kSteps - kS1;
#pragma unroll
          for (int rt = (st - kS1) * kRT / kS2; rt < (st - kS1 + 1) * kRT / kS2; ++rt) item_split(rt, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (with_loads) asm volatile("" ::: "memory");
    if (soft) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) item_split(rt, kKT - 1);
    }
  };

  if (ntiles > 0) {
    // Loads go out in the order K(0) V(0) K(1) V(1) ...: the prologue takes
    // K(0 .. kSlots - 1) and V(0 .. kSlots - 2); iteration i refills V(i - 2 +
    // kSlots), then K(i - 1 + kSlots).
    for (int i = 0; i < kSlots && i < ntiles; ++i) refill(i >= 1 ? i - 1 : ntiles, i);
    if (ntiles <= kSlots - 1) refill(ntiles - 1, ntiles);  // a short stream: its last values too
    // the start of iteration it: K(it) and V(it - 1) have landed (later loads
    // may stay in flight), then the freed slots are refilled
    auto sync = [&](int it) __attribute__((always_inline)) {
      if (it < ntiles) {
        if (it >= 2 && it - 2 + kSlots < ntiles) {
          wait_vmem<kIPW * 2 * (kSlots - 2)>();
        } else {
          const int kmax = min(ntiles - 1, it >= 2 ? it - 2 + kSlots : kSlots - 1);
          const int vmax = min(ntiles - 1, it >= 2 ? it - 3 + kSlots : kSlots - 2);
          wait_vm_upto(kIPW * (max(0, kmax - it) + max(0, vmax - it + 1)));
        }
      } else {
        wait_vmem<0>();  // V(ntiles - 1), the last load
      }
      lds_barrier();
    };
    // stage 0: scores and softmax alone
    sync(0);
    scores(0);
    mask_scores(0);
    soft_all();
    rescale();
    // iteration it: scores of stage it, then P.V of stage it - 1 with the
    // softmax of stage it
    for (int it = 1; it < ntiles; ++it) {
      sync(it);
      fetch_pages(it - 2 + kSlots, it - 1 + kSlots);
      scores(it);
      const bool spread = it - 2 + kSlots < ntiles && prepare(it - 2 + kSlots, it - 1 + kSlots);
      mask_scores(it);
      pv_product(it - 1, spread, true);
      rescale();
    }
    sync(ntiles);
    pv_product(ntiles - 1, false, false);
  }

#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const float l_tot = acc_l[rt][0];
    if (!ok[rt]) continue;
    const int t = Rr[rt] / G, hl = Rr[rt] % G;
    const size_t qoff = ((static_cast<size_t>(b) * N + t) * Hq + g * G + hl) * D;
    wide_row_store<TO, D>(final_out, acc[rt], m_run[rt], l_tot, lg, out + qoff, ws_acc, ws_ml,
                          pslot * rows + Rr[rt]);
  }
}

// Stream decomposition of a layer without a window.  The tiles of every
// (sequence, kv head) unit -- its context keys in tiles of 32, then its node
// tiles -- are laid end to end in unit order j = g * B + b, and workgroup w
// takes the contiguous share [w * per, (w + 1) * per) of that sequence.  Every
// workgroup streams the same number of tiles, whatever the mix of context
// lengths, so the grid ends together.  A workgroup walks the units its share
// touches as segments; a unit covered by one segment is written out directly,
// otherwise each segment leaves a partial in slot w + j (unique, because
// shares are disjoint and ordered) for the merge.
constexpr int kMaxSeqs = 4 * kThreads - 1;  // sequences the stream prefix covers

struct StreamLayout {
  int total;  // tiles over all units
  int per;    // tiles per workgroup
};

// tiles of sequence b's units and their start offsets: s_pref[b] = tiles of
// sequences before b (one kv head each), filled for b = 0..B
__device__ __forceinline__ void stream_prefix(const int32_t* ctx_len, int max_ctx, int B, int N,
                                              int* s_pref, int* s_ctx = nullptr) {
  const int tid = threadIdx.x;
  const int ntn = (N + kTile - 1) / kTile;
  // each thread owns up to 4 consecutive sequences; the four context lengths
  // are loaded unconditionally (the last sequence's past B), so they are in
  // flight together rather than one round trip after another
  int raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = ctx_len[min(tid * 4 + i, B - 1)];
  int own[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = tid * 4 + i;
    int tl = 0;
    if (b < B) {
      const int ctx = min(max(raw[i], 0), max_ctx);
      if (s_ctx) s_ctx[b] = ctx;
      tl = (ctx + kTile - 1) / kTile + ntn;
    }
    own[i] = tl;
    sum += tl;
  }
  // inclusive scan of the per-thread sums over the workgroup
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if ((tid & 63) >= off) incl += v;
  }
  __shared__ int s_wave[kWaves];
  if ((tid & 63) == 63) s_wave[tid >> 6] = incl;
  __syncthreads();
  int before = incl - sum;
  for (int w = 0; w < (tid >> 6); ++w) before += s_wave[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = tid * 4 + i;
    if (b <= B) s_pref[b] = before;
    before += own[i];
  }
  __syncthreads();
}

// Shares of the stream layout.  Workgroups w and w + nwg / 2 run on the same
// CU, and the first one's loads are served ahead of the second's; workgroup w
// runs on XCD w % 8, and the odd XCDs stream a little slower than the even
// ones.  With a grid of a multiple of 4 workgroups, the first of a CU pair
// takes pm thousandths of the pair's tiles, and workgroups on even XCDs take
// xm thousandths of their class's average (pm = xm = 1000 / 2 and 1000:
// equal shares).  Shares are contiguous and ordered by w; the four sizes are
// those of (first, even), (first, odd), (second, even), (second, odd).
struct ShareSizes {
  bool weighted;
  int eq;                  // equal share, when not weighted
  int fe, fo, se, so, H;  // sizes and pairs per half
};

__device__ __forceinline__ ShareSizes share_sizes(int nwg, int total, int pm, int xm) {
  ShareSizes z;
  z.weighted = (nwg & 3) == 0 && (pm != 500 || xm != 1000);
  z.eq = (total + nwg - 1) / nwg;
  z.H = nwg >> 1;
  const int pp = z.weighted ? (total + z.H - 1) / z.H : 0;  // tiles per CU pair
  const int A = static_cast<int>((static_cast<long long>(pp) * pm + 500) / 1000);
  const int Bs = pp - A;
  z.fe = static_cast<int>((static_cast<long long>(A) * xm + 500) / 1000);
  z.fo = 2 * A - z.fe;
  z.se = static_cast<int>((static_cast<long long>(Bs) * xm + 500) / 1000);
  z.so = 2 * Bs - z.se;
  return z;
}

// share of workgroup w: tiles [x, y) of `total`
__device__ __forceinline__ int2 share_at(const ShareSizes& z, int w, int total) {
  int r0, len;
  if (!z.weighted) {
    r0 = w * z.eq;
    len = z.eq;
  } else if (w < z.H) {
    r0 = (w >> 1) * (z.fe + z.fo) + (w & 1) * z.fe;
    len = (w & 1) ? z.fo : z.fe;
  } else {
    const int v = w - z.H;
    r0 = (z.H >> 1) * (z.fe + z.fo) + (v >> 1) * (z.se + z.so) + (v & 1) * z.se;
    len = (v & 1) ? z.so : z.se;
  }
  r0 = min(r0, total);
  return make_int2(r0, min(total, r0 + len));
}

// workgroup whose share holds tile x (0 <= x < total)
__device__ __forceinline__ int owner_of(const ShareSizes& z, int x) {
  if (!z.weighted) return x / z.eq;
  const int first = (z.H >> 1) * (z.fe + z.fo);  // tiles of the first workgroups of the pairs
  if (x < first) {
    const int k = x / (z.fe + z.fo);
    return 2 * k + (x - k * (z.fe + z.fo) >= z.fe ? 1 : 0);
  }
  // the second workgroups hold the rest: x < H * (tiles per pair), so se + so > 0
  const int y = x - first;
  const int k = y / (z.se + z.so);
  return z.H + 2 * k + (y - k * (z.se + z.so) >= z.se ? 1 : 0);
}

// workgroups per CU the stream kernel's register budget is sized for (fp32
// inputs from D = 128 on need more than half the register file)
template <typename T, int D>
constexpr int stream_min_wg() {
  return (sizeof(T) == 4 && D >= 128) ? 1 : TV_ATTN_MIN_WG;
}

template <typename T, typename TO, int D>
__global__ __launch_bounds__(kThreads, (stream_min_wg<T, D>())) void attn_stream_kernel(
    const T* __restrict__ q, const T* __restrict__ kn, const T* __restrict__ vn,
    const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ bt,
    int max_blocks, int num_blocks, const int32_t* __restrict__ ctx_len, int max_ctx,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ pos, int B, int N, int Hq,
    int Hkv, int G, int rows, float scale_log2, int pm, int xm, TO* __restrict__ out,
    float* __restrict__ ws_acc, float2* __restrict__ ws_ml) {
  using C = Cfg<T, D>;
  __shared__ __align__(1024) unsigned char kring[C::kSlots * C::kTileBytes];
  __shared__ __align__(1024) unsigned char vring[C::kSlots * C::kTileBytes];
  __shared__ int s_pages[kMaxPages];
  __shared__ int s_pos[TV_MAX_NODES];  // node positions: read only under a window, never here
  __shared__ int s_pref[kMaxSeqs + 1];
  __shared__ int s_ctx[kMaxSeqs + 1];

  const int ntn = (N + kTile - 1) / kTile;
  stream_prefix(ctx_len, max_ctx, B, N, s_pref, s_ctx);
  const int tb_all = s_pref[B];  // tiles of one kv head over all sequences
  const int total = tb_all * Hkv;
  const int w = blockIdx.x;
  const int2 share = share_at(share_sizes(gridDim.x, total, pm, xm), w, total);
  int cur = share.x;
  const int r1 = share.y;

  while (cur < r1) {
    // units are head-major, j = g * B + b: at any moment the workgroups stream
    // different sequences' pages rather than the heads of one page block
    const int g = cur / tb_all;
    const int rem = cur - g * tb_all;
    int b = 0;
    {
      int lo = 0, hi = B - 1;  // last sequence starting at or before rem
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= rem) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
    }
    const int tiles_b = s_pref[b + 1] - s_pref[b];
    const int us = g * tb_all + s_pref[b];  // first tile of unit (b, g)
    const int t0 = cur - us;
    const int t1 = min(tiles_b, r1 - us);
    const int ctx = s_ctx[b];
    const int nct = tiles_b - ntn;  // context tiles of the unit
    const int k0 = min(min(t0, nct) * kTile, ctx);
    const int k1 = min(min(t1, nct) * kTile, ctx);
    const int n0 = max(t0, nct) - nct;
    const int n1 = max(t1, nct) - nct;

    __syncthreads();  // the previous segment is done with every LDS buffer
    const int32_t* pos_b = pos + static_cast<size_t>(b) * N;
    const int2 prng = make_int2(0, 0);  // position range: only windows use it
    // the page indices, then the query rows, go out together; the page
    // stores wait only for the former
    const int32_t* bt_b = bt + static_cast<size_t>(b) * max_blocks;
    const int p0 = k0 >> 4;
    const int npages = k1 > k0 ? ((k1 - 1) >> 4) - p0 + 1 : 0;
    const PageLoads<kThreads, kMaxPages> pl = pages_issue<kThreads, kMaxPages>(bt_b, p0, npages);
    const RowIn<T, D> ri = row_in<T, D>(q, pos_b, anc, b, g, 0, N, Hq, G, rows);
    pages_store<kThreads, kMaxPages>(s_pages, pl, num_blocks);

    attn_segment<T, TO, D, 1, kMaxPages>(ri, kn, vn, kc, vc, bt_b, num_blocks, anc, pos_b, N, Hq, Hkv, G, rows,
                           0, scale_log2, b, g, 0, k0, k1, n0, n1, prng,
                           t0 == 0 && t1 == tiles_b, static_cast<size_t>(w) + g * B + b, out,
                           ws_acc, ws_ml, kring, vring, s_pages, s_pos);
    cur = us + t1;
  }
}

// Merge of the stream layout: unit (b, g) covers tiles [us, us + tiles_b);
// its segments belong to workgroups us / per .. (us + tiles_b - 1) / per and
// sit in slots w + j.  A unit with one segment was written out directly.
// A block merges kMergeRows rows of one unit, 16 threads per row, each thread
// D / 64 groups of 4 columns.
constexpr int kMergeRows = 16;

template <typename TO, int D>
__global__ __launch_bounds__(256) void attn_merge_stream_kernel(
    const int32_t* __restrict__ ctx_len, int max_ctx, int B, int N, int Hq, int Hkv, int G,
    int rows, int nwg, int pm, int xm, const float* __restrict__ ws_acc,
    const float2* __restrict__ ws_ml, TO* __restrict__ out) {
  constexpr int kV = D / 64;  // float4 column groups per thread
  static_assert(kV >= 1 && 16 * kMergeRows == 256, "merge layout");
  __shared__ int s_pref[kMaxSeqs + 1];
  const int chunks = (rows + kMergeRows - 1) / kMergeRows;
  const int j = blockIdx.x / chunks;  // head-major unit rank g * B + b
  const int chunk = blockIdx.x % chunks;
  const int g = j / B;
  const int b = j % B;
  stream_prefix(ctx_len, max_ctx, B, N, s_pref);
  const int tb_all = s_pref[B];
  const int total = tb_all * Hkv;
  const int tiles_b = s_pref[b + 1] - s_pref[b];
  const int us = g * tb_all + s_pref[b];
  const ShareSizes z = share_sizes(nwg, total, pm, xm);
  const int w_lo = owner_of(z, us);
  const int w_hi = owner_of(z, us + tiles_b - 1);
  if (w_lo == w_hi) return;
  const int R = chunk * kMergeRows + threadIdx.x / 16;
  if (R >= rows) return;
  const int c0 = (threadIdx.x % 16) * 4;
  float mx = -INFINITY, L = 0.f;
  float4 o[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  // partials four at a time: every load of a group is issued before any is used
  constexpr int kP = 4;
  for (int w0 = w_lo; w0 <= w_hi; w0 += kP) {
    float2 ml[kP];
    float4 a[kP][kV];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      const int w = w0 + p;
      ml[p] = make_float2(-INFINITY, 0.f);
      if (w <= w_hi) {
        const int2 sh = share_at(z, w, total);
        if (sh.x < sh.y) {  // an empty share left no partial
          const size_t ub = (static_cast<size_t>(w) + j) * rows + R;
          ml[p] = ws_ml[ub];
#pragma unroll
          for (int k = 0; k < kV; ++k) a[p][k] = *reinterpret_cast<const float4*>(ws_acc + ub * D + c0 + 64 * k);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      if (ml[p].x == -INFINITY) continue;  // no partial, or it saw no key of the row
      const float m_new = fmaxf(mx, ml[p].x);
      const float c_old = fast_exp2(mx - m_new);
      const float c_new = fast_exp2(ml[p].x - m_new);
      // explicit fmaf: both output types' instantiations round alike
      L = __builtin_fmaf(ml[p].y, c_new, L * c_old);
#pragma unroll
      for (int k = 0; k < kV; ++k) {
        o[k].x = __builtin_fmaf(a[p][k].x, c_new, o[k].x * c_old);
        o[k].y = __builtin_fmaf(a[p][k].y, c_new, o[k].y * c_old);
        o[k].z = __builtin_fmaf(a[p][k].z, c_new, o[k].z * c_old);
        o[k].w = __builtin_fmaf(a[p][k].w, c_new, o[k].w * c_old);
      }
      mx = m_new;
    }
  }
  const float inv = 1.0f / L;
  const int t = R / G, hl = R % G;
  TO* op = out + ((static_cast<size_t>(b) * N + t) * Hq + g * G + hl) * D + c0;
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    if constexpr (sizeof(TO) == 2) {
      uint2 wv;
      wv.x = static_cast<uint32_t>(f32_to_bf16(o[k].x * inv)) |
             (static_cast<uint32_t>(f32_to_bf16(o[k].y * inv)) << 16);
      wv.y = static_cast<uint32_t>(f32_to_bf16(o[k].z * inv)) |
             (static_cast<uint32_t>(f32_to_bf16(o[k].w * inv)) << 16);
      *reinterpret_cast<uint2*>(op + 64 * k) = wv;
    } else {
      *reinterpret_cast<float4*>(op + 64 * k) =
          make_float4(o[k].x * inv, o[k].y * inv, o[k].z * inv, o[k].w * inv);
    }
  }
}

// Log-sum-exp merge of the split partials of sequences that used more than
// one split.  Thread = 4 consecutive output columns of one row.
template <typename TO, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const int32_t* __restrict__ ctx_len, int max_ctx, const int32_t* __restrict__ pos, int N,
    int Hq, int Hkv, int G, int rows, int nsplit_max, int split_tokens, int window,
    const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml, TO* __restrict__ out) {
  constexpr int kTpr = D / 4;       // threads per row
  constexpr int kRpb = 256 / kTpr;  // rows per block
  __shared__ int2 s_rng;
  const int chunks = (rows + kRpb - 1) / kRpb;
  const int bg = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int32_t* pos_b = pos + static_cast<size_t>(b) * N;
  const int2 prng = tree_pos_range(pos_b, N, &s_rng);
  const SeqPlan sp = seq_plan(ctx_len[b], max_ctx, window, prng.x, nsplit_max, split_tokens);
  if (sp.nsplit == 1) return;
  const int R = chunk * kRpb + threadIdx.x / kTpr;
  if (R >= rows) return;
  const int d0 = (threadIdx.x % kTpr) * 4;
  const size_t ub0 = (static_cast<size_t>(b) * Hkv + g) * nsplit_max * rows + R;
  // one pass: running max, rescaling the running sums when it moves
  float mx = -INFINITY, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = 0; s < sp.nsplit; ++s) {
    const size_t ub = ub0 + static_cast<size_t>(s) * rows;
    const float2 ml = ws_ml[ub];
    const float4 a = *reinterpret_cast<const float4*>(ws_acc + ub * D + d0);
    if (ml.x == -INFINITY) continue;  // this split saw no key of the row
    const float m_new = fmaxf(mx, ml.x);
    const float c_old = fast_exp2(mx - m_new);  // 0 while mx is still -inf
    const float c_new = fast_exp2(ml.x - m_new);
    // explicit fmaf: both output types' instantiations round alike
    L = __builtin_fmaf(ml.y, c_new, L * c_old);
    o.x = __builtin_fmaf(a.x, c_new, o.x * c_old);
    o.y = __builtin_fmaf(a.y, c_new, o.y * c_old);
    o.z = __builtin_fmaf(a.z, c_new, o.z * c_old);
    o.w = __builtin_fmaf(a.w, c_new, o.w * c_old);
    mx = m_new;
  }
  const float inv = 1.0f / L;
  const int t = R / G, hl = R % G;
  TO* op = out + ((static_cast<size_t>(b) * N + t) * Hq + g * G + hl) * D + d0;
  if constexpr (sizeof(TO) == 2) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16(o.x * inv)) | (static_cast<uint32_t>(f32_to_bf16(o.y * inv)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16(o.z * inv)) | (static_cast<uint32_t>(f32_to_bf16(o.w * inv)) << 16);
    *reinterpret_cast<uint2*>(op) = w;
  } else {
    *reinterpret_cast<float4*>(op) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

template <typename T, typename TO, int D>
hipError_t launch_typed(const AttnPlan& pl, const void* q, const void* k_node, const void* v_node,
                        const void* k_cache, const void* v_cache, const int32_t* block_table,
                        int max_blocks, int num_blocks, const int32_t* ctx_len, int max_ctx,
                        const uint64_t* anc, const int32_t* pos, int B, int N, int Hq, int Hkv,
                        int window, float scale, void* out, void* ws, hipStream_t stream) {
  const long long units = static_cast<long long>(B) * Hkv * pl.nsplit;
  const long long grid = (units + 7) / 8 * 8 * pl.row_groups;
  float* ws_acc = nullptr;
  float2* ws_ml = nullptr;
  if (pl.nsplit > 1) {
    ws_acc = static_cast<float*>(ws);
    ws_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                      static_cast<size_t>(B) * Hkv * pl.nsplit * pl.rows * D * 4);
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  constexpr int kRpb = 256 / (D / 4);
  const unsigned merge_grid = static_cast<unsigned>(B) * Hkv * ((pl.rows + kRpb - 1) / kRpb);
  if (pl.stream_wg > 0) {
    ws_acc = static_cast<float*>(ws);
    const size_t slots = static_cast<size_t>(pl.stream_wg) + static_cast<size_t>(B) * Hkv - 1;
    ws_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + slots * pl.rows * D * 4);
    hipLaunchKernelGGL((attn_stream_kernel<T, TO, D>), dim3(pl.stream_wg), dim3(kThreads), 0,
                       stream, static_cast<const T*>(q), static_cast<const T*>(k_node),
                       static_cast<const T*>(v_node), static_cast<const T*>(k_cache),
                       static_cast<const T*>(v_cache), block_table, max_blocks, num_blocks,
                       ctx_len, max_ctx, anc, pos, B, N, Hq, Hkv, pl.G, pl.rows, scale_log2,
                       pl.stream_pm, pl.stream_xm, static_cast<TO*>(out), ws_acc, ws_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned sm_grid =
        static_cast<unsigned>(B) * Hkv * ((pl.rows + kMergeRows - 1) / kMergeRows);
    hipLaunchKernelGGL((attn_merge_stream_kernel<TO, D>), dim3(sm_grid), dim3(256), 0, stream,
                       ctx_len, max_ctx, B, N, Hq, Hkv, pl.G, pl.rows, pl.stream_wg, pl.stream_pm,
                       pl.stream_xm, ws_acc, ws_ml, static_cast<TO*>(out));
    return hipGetLastError();
  }
  if constexpr (sizeof(T) == 2) {
    if (pl.rows > kRows) {
      // wide query tiles: 16 kRT rows per wave
      constexpr int kRowsW = 16 * wide_tiles<D>() * kWideWaves;
      const int rgw = (pl.rows + kRowsW - 1) / kRowsW;
      const long long gridw = (units + 7) / 8 * 8 * rgw;
      hipLaunchKernelGGL((attn_wide_kernel<TO, D>), dim3(static_cast<unsigned>(gridw)),
                         dim3(64 * kWideWaves), 0, stream, static_cast<const T*>(q),
                         static_cast<const T*>(k_node), static_cast<const T*>(v_node),
                         static_cast<const T*>(k_cache), static_cast<const T*>(v_cache),
                         block_table, max_blocks, num_blocks, ctx_len, max_ctx, anc, pos, N, Hq,
                         Hkv, pl.G, pl.rows, rgw, pl.nsplit, pl.split_tokens, window, scale_log2,
                         static_cast<int>(units), static_cast<TO*>(out), ws_acc, ws_ml);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || pl.nsplit == 1) return e;
      hipLaunchKernelGGL((attn_merge_kernel<TO, D>), dim3(merge_grid), dim3(256), 0, stream, ctx_len,
                         max_ctx, pos, N, Hq, Hkv, pl.G, pl.rows, pl.nsplit, pl.split_tokens, window,
                         ws_acc, ws_ml, static_cast<TO*>(out));
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_split_kernel<T, TO, D>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads * split_teams<T, D>()),
                     0, stream, static_cast<const T*>(q), static_cast<const T*>(k_node),
                     static_cast<const T*>(v_node), static_cast<const T*>(k_cache),
                     static_cast<const T*>(v_cache), block_table, max_blocks, num_blocks, ctx_len,
                     max_ctx, anc, pos, N, Hq, Hkv, pl.G, pl.rows, pl.row_groups, pl.nsplit,
                     pl.split_tokens, window, scale_log2, static_cast<int>(units),
                     static_cast<TO*>(out), ws_acc, ws_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  hipLaunchKernelGGL((attn_merge_kernel<TO, D>), dim3(merge_grid), dim3(256), 0, stream, ctx_len, max_ctx,
                     pos, N, Hq, Hkv, pl.G, pl.rows, pl.nsplit, pl.split_tokens, window, ws_acc,
                     ws_ml, static_cast<TO*>(out));
  return hipGetLastError();
}

}  // namespace

#ifndef TV_ATTN_MIN_SPLIT
#define TV_ATTN_MIN_SPLIT 2048  // keys per split at least (partials stay small)
#endif
#ifndef TV_ATTN_TARGET_WG
#define TV_ATTN_TARGET_WG 4096  // workgroups the split plan aims for
#endif

#ifndef TV_ATTN_STREAM_WG_PER_CU
#define TV_ATTN_STREAM_WG_PER_CU 2  // resident workgroups per CU in the stream layout
#endif
#ifndef TV_ATTN_PAIR_PM
#define TV_ATTN_PAIR_PM 535  // thousandths of a CU's tiles for the first of its two workgroups
#endif
#ifndef TV_ATTN_XCD_PM
#define TV_ATTN_XCD_PM 1050  // thousandths of the average share for workgroups on even XCDs
#endif
static_assert(TV_ATTN_PAIR_PM >= 500 && TV_ATTN_PAIR_PM < 1000, "pair weight");
static_assert(TV_ATTN_XCD_PM >= 500 && TV_ATTN_XCD_PM <= 1500, "XCD weight");
#ifndef TV_ATTN_STREAM_MIN_TILES
#define TV_ATTN_STREAM_MIN_TILES 16  // key tiles per stream workgroup while the grid fills the chip
#endif

int device_cus() {
  static std::atomic<int> cached[64];  // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int device_xcds() {
  static std::atomic<int> cached[64];  // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) n = -1;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

AttnPlan attn_plan(int B, int N, int Hq, int Hkv, int D, int max_ctx_len, int window) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.rows = p.G * N;
  p.row_groups = (p.rows + kRows - 1) / kRows;
  // Global layers whose rows fit one workgroup use the stream layout: every
  // workgroup streams the same number of key tiles, so batches of mixed
  // context length end together.  Partials: one slot per (workgroup, unit)
  // pair a share touches, at most workgroups + units - 1.
  const long long units = static_cast<long long>(B) * Hkv;
  const long long tiles =
      units * ((static_cast<long long>(max_ctx_len) + kTile - 1) / kTile + (N + kTile - 1) / kTile);
  if (TV_ATTN_STREAM_WG_PER_CU > 0 && window <= 0 && p.row_groups == 1 && B >= 1 && B <= kMaxSeqs && tiles < (1ll << 30)) {
    long long wg = static_cast<long long>(TV_ATTN_STREAM_WG_PER_CU) * device_cus();
    // tiles per workgroup: at least TV_ATTN_STREAM_MIN_TILES while the grid
    // fills the chip (the partials stay small next to the keys streamed);
    // fewer, down to 2, for small batches, whose time is latency
    long long per = (tiles + wg - 1) / wg;
    if (per > TV_ATTN_STREAM_MIN_TILES) per = TV_ATTN_STREAM_MIN_TILES;
    if (per < 2) per = 2;
    const long long by_work = (tiles + per - 1) / per;
    if (wg > by_work) wg = by_work;
    if (wg < 1) wg = 1;
    p.stream_wg = static_cast<int>(wg);
    // a full grid of two workgroups per CU pairs workgroup w with w + CUs; the
    // pair and XCD weights were measured on 256 CUs in 8 XCDs and apply only
    // there (equal shares elsewhere)
    bool full = TV_ATTN_STREAM_WG_PER_CU == 2 && wg == 2ll * device_cus() && device_cus() == 256 &&
                device_xcds() == 8;
    // a share spans at most the page cache's worth of key tiles (weighted
    // shares run up to about 12% over the average), so every segment's page
    // indices fit the cache: larger batches get more workgroups, with equal
    // shares, rather than a block-table read per refill
    const long long cap = static_cast<long long>(kMaxPages) * 16 / kTile;
    const long long avg = (tiles + wg - 1) / wg;
    if ((full ? avg * 115 / 100 + 1 : avg) > cap) {
      wg = (tiles + cap - 1) / cap;
      full = false;
      p.stream_wg = static_cast<int>(wg);
    }
    p.stream_pm = full ? TV_ATTN_PAIR_PM : 500;
    p.stream_xm = full ? TV_ATTN_XCD_PM : 1000;
    p.nsplit = 1;
    p.split_tokens = kTile;
    p.ws_bytes = static_cast<size_t>(wg + units - 1) * p.rows * (static_cast<size_t>(D) * 4 + 8);
    return p;
  }
  const int range = window > 0 ? (max_ctx_len < window ? max_ctx_len : window) : max_ctx_len;
  // aim for a few thousand workgroups, but keep each split long enough that
  // its fp32 partials stay small next to the keys it streams
  const long long units_rg = units * p.row_groups;
  long long want = (TV_ATTN_TARGET_WG + units_rg - 1) / units_rg;
  const int min_split = TV_ATTN_MIN_SPLIT;
  long long cap = (range + min_split - 1) / min_split;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  int st = static_cast<int>((range + want - 1) / want);
  st = (st + kTile - 1) / kTile * kTile;
  if (st < kTile) st = kTile;
  // a split's page indices must fit the page cache (a window start or split
  // start inside a page adds one page): otherwise every load past the cache
  // would wait for a block-table read
  constexpr int kMaxSplit = (kSplitPages - 2) * 16 / kTile * kTile;
  if (st > kMaxSplit) st = kMaxSplit;
  p.split_tokens = st;
  p.nsplit = range > 0 ? (range + st - 1) / st : 1;
  p.ws_bytes = p.nsplit > 1
                   ? static_cast<size_t>(B) * Hkv * p.nsplit * p.rows * (static_cast<size_t>(D) * 4 + 8)
                   : 0;
  return p;
}

hipError_t launch_attn(const AttnPlan& plan, const void* q, const void* k_node, const void* v_node,
                       const void* k_cache, const void* v_cache, const int32_t* block_table,
                       int max_blocks, int num_blocks, const int32_t* ctx_len, int max_ctx_len,
                       const uint64_t* anc, const int32_t* pos, int B, int N, int Hq, int Hkv,
                       int D, int window, float scale, tv_dtype dtype, tv_dtype out_dtype,
                       void* out, void* ws, hipStream_t stream) {
#define TV_ATTN_CASE(TYPE, OTYPE, DIM)                                                          \
  return launch_typed<TYPE, OTYPE, DIM>(plan, q, k_node, v_node, k_cache, v_cache, block_table, \
                                        max_blocks, num_blocks, ctx_len, max_ctx_len, anc, pos, \
                                        B, N, Hq, Hkv, window, scale, out, ws, stream)
#define TV_ATTN_DIMS(TYPE, OTYPE)               \
  if (D == 64) TV_ATTN_CASE(TYPE, OTYPE, 64);   \
  if (D == 128) TV_ATTN_CASE(TYPE, OTYPE, 128); \
  if (D == 256) TV_ATTN_CASE(TYPE, OTYPE, 256);
  if (dtype == TV_BF16 && out_dtype == TV_BF16) { TV_ATTN_DIMS(uint16_t, uint16_t) }
  if (dtype == TV_BF16 && out_dtype == TV_F32) { TV_ATTN_DIMS(uint16_t, float) }
  if (dtype == TV_F32 && out_dtype == TV_F32) { TV_ATTN_DIMS(float, float) }
#undef TV_ATTN_DIMS
#undef TV_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace tv
