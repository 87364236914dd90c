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
// the log-sum-exp over the vocabulary (fp64) and the K largest logits (ties
// to the lower token id), in one pass (an HBM stream).  tree_build_kernel: one
// wave per sequence runs the queue in registers; a candidate's push counter is
// its slot, so "equal scores in push order" is "equal scores, lower slot".
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kTopkThreads = 512;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kKMax = TV_TREE_MAX_TOPK;  // longest wave list (lanes 0 .. K - 1)

// order of the top-k selection: larger value first, then lower index
// (bitwise operators: straight-line compares, no short-circuit branches)
__device__ __forceinline__ bool cand_before(float av, int ai, float bv, int bi) {
  return (av > bv) | ((av == bv) & (ai < bi));
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
// values, the latter correctly rounded to fp32 (the fp64 log-sum-exp, rounded
// once).  Each thread scans 16-byte chunks c = tid, tid + 512, ... keeping a
// running max m.  An element more than kBig below the workgroup's running max
// (shared through LDS after every pass) adds its exp in fp32 to a running sum
// s: all of them together weigh at most V e^-kBig of the row's sum (the row
// maximum alone weighs 1), so the fp32 rounding there stays far below fp32's
// resolution of the result.  The larger elements are queued in LDS, one value
// per entry (the input's own bits), and once per pass the wave sums their exp
// in fp64, 64 at a time (one per lane), against a wave-uniform reference; the
// next pass's loads are in flight meanwhile.  Each wave keeps one sorted list
// of its K best (lane k < K holds entry k): an element is a candidate only if
// it beats the list's last entry, which the whole wave knows, so after the
// first few chunks a chunk costs a compare and a ballot; candidates enter one
// at a time by a lane-parallel insertion, element slot by element slot, and
// after each insertion the ones still waiting are checked again against the
// new last entry.  The waves'
// lists and sums merge at the end.
constexpr float kBig = 22.0f;  // natural-log distance below the running max summed in fp32
constexpr int kU = 4;          // 16-byte chunks per thread and pass

// order-preserving map of a float onto a signed int (for an LDS atomicMax)
__device__ __forceinline__ int f2ord(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float ord2f(int i) { return __int_as_float(i >= 0 ? i : i ^ 0x7fffffff); }

// one DPP lane exchange of a 32-bit value (a lane whose source does not exist
// keeps `old`)
template <int kCtrl>
__device__ __forceinline__ int dpp(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, kCtrl, 0xf, 0xf, false);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// the wave's maximum, in every lane: the rows of 16 lanes reduce by quad
// exchanges and rotations, then the four row maxima are read out
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp<0xb1>(0, __float_as_int(v))));   // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(dpp<0x4e>(0, __float_as_int(v))));   // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(dpp<0x124>(0, __float_as_int(v))));  // row_ror 4
  v = fmaxf(v, __int_as_float(dpp<0x128>(0, __float_as_int(v))));  // row_ror 8
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

template <typename T>
__global__ __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(4))) void draft_topk_kernel(const T* __restrict__ logits,
                                                                  int V, int K,
                                                                  int32_t* __restrict__ cand_tok,
                                                                  float* __restrict__ cand_lp) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr int nw = kTopkThreads / 64;
  constexpr int E = 16 / static_cast<int>(sizeof(T));  // elements per chunk
  // Two queues per wave.  Chunks: a chunk with an element at or above its cut
  // (the lane's cut when the chunk was absorbed) is queued whole, with that
  // cut; a pass queues at most 64 * kU and a drain leaves at most 63.
  // Elements: the queued chunks are split 64 at a time, their elements at or
  // above the cut queued one per entry (the input's bits) and summed in fp64,
  // 64 at a time.  The 64 entries past each queue are where the lanes with
  // nothing to queue write.
  constexpr int kCQ = 64 * kU + 63;
  constexpr int kEQ = 64 * E + 63;
  __shared__ u32x4_t s_qc[nw][kCQ + 64];  // queued chunks
  __shared__ float s_qcut[nw][kCQ + 64];  // and their cuts
  __shared__ T s_qe[nw][kEQ + 64];        // queued elements
  __shared__ int s_rowmax;   // the workgroup's running max (order-preserving int)
  const size_t row = blockIdx.x;
  const T* p = logits + row * static_cast<size_t>(V);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_rowmax = f2ord(-INFINITY);
  __syncthreads();

  float wv = -INFINITY;  // this lane's entry of the wave list (lanes < K)
  int wi = 0x7fffffff;
  float thr = -INFINITY;  // the list's entry K - 1, or the floor if that is lower (wave-uniform)
  int thr_i = 0x7fffffff;
  // a value at least K elements of the wave reach (found in the first pass):
  // nothing below it can enter the list
  float floor_v = -INFINITY;
  // offer the elements x[k] (index i0 + k) of the lanes with `ok` set to the
  // wave list, element slot by element slot; every lane of the wave calls it
  auto offer = [&](const float* x, int n, bool ok, int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < n; ++k) {
      uint64_t todo = __ballot(ok && x[k] >= thr);
      while (todo != 0ull) {
        const int src = __ffsll(static_cast<unsigned long long>(todo)) - 1;
        todo &= todo - 1ull;
        const float cv = readlane_f(x[k], src);
        const int ci = __builtin_amdgcn_readlane(i0, src) + k;
        if (!cand_before(cv, ci, thr, thr_i)) continue;  // a tie with a lower index
        // entries after the insertion point move down one lane (K <= 16: row 0)
        const uint64_t worse = __ballot(lane < K && cand_before(cv, ci, wv, wi));
        const int pos = __ffsll(static_cast<unsigned long long>(worse)) - 1;
        const float up_v = __int_as_float(dpp<0x111>(__float_as_int(wv), __float_as_int(wv)));  // row_shr 1
        const int up_i = dpp<0x111>(wi, wi);
        if (lane < K && lane >= pos) {
          wv = lane == pos ? cv : up_v;
          wi = lane == pos ? ci : up_i;
        }
        thr = readlane_f(wv, K - 1);
        thr_i = __builtin_amdgcn_readlane(wi, K - 1);
        if (thr < floor_v) {
          thr = floor_v;
          thr_i = 0x7fffffff;
        }
        todo &= __ballot(ok && x[k] >= thr);
      }
    }
  };
  float m = -INFINITY, s = 0.0f;  // running max and fp32 sum of the small elements' exp(x - m)
  float base = -INFINITY;         // the workgroup's max as last seen
  double S = 0.0;                 // fp64 sum of the queued elements' exp(x - R)
  float R = -INFINITY;            // its reference (wave-uniform, never below a queued element)
  int cq = 0, eq = 0;             // the wave's queue lengths (wave-uniform)

  auto to_q = [](float x) -> T {
    if constexpr (sizeof(T) == 2) return static_cast<T>(__float_as_uint(x) >> 16);
    else return x;
  };
  auto from_q = [](T q) -> float {
    if constexpr (sizeof(T) == 2) return __uint_as_float(static_cast<uint32_t>(q) << 16);
    else return q;
  };
  auto unpack = [](const u32x4_t raw, float* x) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(raw[k] << 16);
        x[2 * k + 1] = __uint_as_float(raw[k] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(raw[k]);
    }
  };
  // the lane's rank among the lanes of `b` (one ballot's lanes)
  auto rank = [&](uint64_t b) __attribute__((always_inline)) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u)));
  };
  // queue the element of the lanes with `big` set (one ballot, no branch)
  auto push_elem = [&](float x, bool big) __attribute__((always_inline)) {
    const uint64_t b = __ballot(big);
    s_qe[wave][big ? eq + rank(b) : kEQ + lane] = to_q(x);
    eq += __popcll(b);
  };
  // queue the chunk of the lanes with `any` set, with its cut
  auto push_chunk = [&](const u32x4_t raw, float cut, bool any) __attribute__((always_inline)) {
    const uint64_t b = __ballot(any);
    const int a = any ? cq + rank(b) : kCQ + lane;
    s_qc[wave][a] = raw;
    s_qcut[wave][a] = cut;
    cq += __popcll(b);
  };
  // every full batch of 64 queued elements (every element, if `all`): their
  // exp in fp64 against R, two batches at a time where there are two (two
  // independent chains); the rest moves to the front of the queue.  R is
  // first raised to the wave's running max, which bounds every queued element
  // (each is at most the running max of the lane that absorbed it).
  auto sum_elems = [&](bool all) __attribute__((always_inline)) {
    if (eq < (all ? 1 : 64)) return;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's queue writes are in
    const float wm = readlane_f(wave_max(m), 0);
    if (wm > R) {
      if (R != -INFINITY) S *= exp(static_cast<double>(R) - static_cast<double>(wm));
      R = wm;
    }
    const double Rd = static_cast<double>(R);
    int h = 0;
    for (; eq - h >= 128; h += 128) {
      const float x0 = from_q(s_qe[wave][h + lane]);
      const float x1 = from_q(s_qe[wave][h + 64 + lane]);
      S += exp(static_cast<double>(x0) - Rd) + exp(static_cast<double>(x1) - Rd);
    }
    while (eq - h >= (all ? 1 : 64)) {
      const int n = min(64, eq - h);
      const float q = from_q(s_qe[wave][h + lane]);
      S += exp(lane < n ? static_cast<double>(q) - Rd : -INFINITY);
      h += n;
    }
    const int left = eq - h;
    if (left > 0) {
      const T v = s_qe[wave][h + lane];  // read by the whole wave before any write
      if (lane < left) s_qe[wave][lane] = v;
    }
    eq = left;
  };
  // every full batch of 64 queued chunks (every chunk, if `all`): their
  // elements at or above the cut go to the element queue, which is summed
  // after each batch; the rest moves to the front of the queue
  auto drain = [&](bool all) __attribute__((always_inline)) {
    if (cq >= (all ? 1 : 64)) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's queue writes are in
      int h = 0;
      while (cq - h >= (all ? 1 : 64)) {
        const int n = min(64, cq - h);
        const u32x4_t raw = s_qc[wave][h + lane];
        const float cut = s_qcut[wave][h + lane];
        float x[E];
        unpack(raw, x);
#pragma unroll
        for (int k = 0; k < E; ++k) push_elem(x[k], lane < n && !(x[k] < cut));
        sum_elems(false);
        h += n;
      }
      const int left = cq - h;
      if (left > 0) {
        const u32x4_t raw = s_qc[wave][h + lane];  // read by the whole wave before any write
        const float cut = s_qcut[wave][h + lane];
        if (lane < left) {
          s_qc[wave][lane] = raw;
          s_qcut[wave][lane] = cut;
        }
      }
      cq = left;
    }
    if (all) sum_elems(true);
  };

  const bool vec = ((static_cast<size_t>(V) * sizeof(T)) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  const int nchunk = vec ? V / E : 0;
  // one chunk: the running max and sums absorb it, and its elements are
  // offered to the wave list.  Called by the whole wave (the list lives in its
  // first K lanes); a lane without a chunk offers nothing.
  auto absorb = [&](const u32x4_t raw, int c, bool valid) __attribute__((always_inline)) {
    float x[E];
    unpack(raw, x);
    float cm = x[0];
#pragma unroll
    for (int k = 1; k < E; ++k) cm = fmaxf(cm, x[k]);
    bool any = false;
    float cut = 0.0f;
    if (valid) {
      const float nm = fmaxf(m, cm);
      cut = fmaxf(nm, base) - kBig;
      float add = 0.0f;
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const bool big = !(x[k] < cut);
        any = any || big;
        if (!big) add += __builtin_amdgcn_exp2f((x[k] - nm) * kLog2e);
      }
      s = (m == -INFINITY ? 0.0f : s * __builtin_amdgcn_exp2f((m - nm) * kLog2e)) + add;
      m = nm;
    }
    push_chunk(raw, cut, any);
    if (__ballot(valid && cm >= thr) != 0ull) offer(x, E, valid, c * E);
  };
  // share the running max: publish the wave's, read the workgroup's
  auto share_max = [&]() __attribute__((always_inline)) {
    const float wm = wave_max(m);
    if (lane == 0) atomicMax(&s_rowmax, f2ord(wm));
    base = fmaxf(base, ord2f(s_rowmax));
  };
  // passes of kU chunks per thread; the loop bounds are wave-uniform (cw =
  // the wave's first chunk of a pass).  The next pass's loads are issued
  // before this one is absorbed (from the same pass again where there is no
  // next: in bounds, unused).
  constexpr int kPass = kU * kTopkThreads;
  const u32x4_t* pc = reinterpret_cast<const u32x4_t*>(p);
  auto full = [&](int c) { return c + 63 + (kU - 1) * kTopkThreads < nchunk; };
  int cw = wave * 64;
  bool have = full(cw);
  {
    // the first pass: the maximum of its chunks is shared before any of them
    // is classified (the running max knows nothing yet); the barrier is
    // reached by every wave, with or without a first pass
    u32x4_t r[kU];
    float lm = -INFINITY;
    if (have) {
#pragma unroll
      for (int u = 0; u < kU; ++u) r[u] = __builtin_nontemporal_load(pc + cw + lane + u * kTopkThreads);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            lm = fmaxf(lm, fmaxf(__uint_as_float(r[u][k] << 16), __uint_as_float(r[u][k] & 0xffff0000u)));
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) lm = fmaxf(lm, __uint_as_float(r[u][k]));
        }
      }
    }
    if (have) {
      // the floor: the K-th largest lane maximum of this pass (one lane
      // leaves per round, so equal maxima count separately)
      float t = lm;
      for (int j = 0; j < K; ++j) {
        floor_v = readlane_f(wave_max(t), 0);
        const uint64_t hb = __ballot(t == floor_v);
        if (lane == __ffsll(static_cast<unsigned long long>(hb)) - 1) t = -INFINITY;
      }
      thr = floor_v;
    }
    lm = wave_max(lm);
    if (lane == 0) atomicMax(&s_rowmax, f2ord(lm));
    __syncthreads();
    base = ord2f(s_rowmax);
    while (have) {
      const int cn = cw + kPass;
      const bool more = full(cn);
      const int cl = more ? cn : cw;
      u32x4_t rn[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) rn[u] = __builtin_nontemporal_load(pc + cl + lane + u * kTopkThreads);
#pragma unroll
      for (int u = 0; u < kU; ++u) absorb(r[u], cw + lane + u * kTopkThreads, true);
      share_max();
      drain(false);
#pragma unroll
      for (int u = 0; u < kU; ++u) r[u] = rn[u];
      cw = cn;
      have = more;
    }
  }
  for (; cw < nchunk; cw += kTopkThreads) {
    const int c = cw + lane;
    const bool ok = c < nchunk;
    const u32x4_t r = __builtin_nontemporal_load(pc + (ok ? c : 0));
    absorb(r, c, ok);
    drain(false);
  }
  // elements past the last whole chunk (or every element without 16-byte
  // rows): all go to the queue; the loop runs while any lane of the wave has one
  for (int v0 = nchunk * E + (tid & ~63); v0 < V; v0 += kTopkThreads) {
    const int v = v0 + lane;
    const float xv = elem(p, v < V ? v : 0);
    const float x = v < V ? xv : -INFINITY;
    m = fmaxf(m, x);
    push_elem(x, v < V);
    sum_elems(false);
    offer(&x, 1, v < V, v);
  }
  drain(true);

  // log-sum-exp over the workgroup, in fp64: the fp32 sums of the small
  // elements (each relative to its lane's max) and the fp64 sums (relative to
  // their wave's reference)
  __shared__ float s_m[nw], s_r[nw];
  __shared__ double s_s[nw], s_big[nw];
  __shared__ float s_lv[nw][kKMax];
  __shared__ int s_li[nw][kKMax];
  float wm = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off, 64));
  double ws = m == -INFINITY ? 0.0 : static_cast<double>(s) * exp(static_cast<double>(m) - static_cast<double>(wm));
  double wb = S;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ws += __shfl_xor(ws, off, 64);
    wb += __shfl_xor(wb, off, 64);
  }
  if (lane < K) {
    s_lv[wave][lane] = wv;
    s_li[wave][lane] = wi;
  }
  if (lane == 0) {
    s_m[wave] = wm;
    s_s[wave] = ws;
    s_r[wave] = R;
    s_big[wave] = wb;
  }
  __syncthreads();
  if (wave != 0) return;
  float gm = -INFINITY;
#pragma unroll
  for (int w = 0; w < nw; ++w) gm = fmaxf(gm, fmaxf(s_m[w], s_r[w]));
  double gs = 0.0;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    if (s_m[w] != -INFINITY) gs += s_s[w] * exp(static_cast<double>(s_m[w]) - static_cast<double>(gm));
    if (s_r[w] != -INFINITY) gs += s_big[w] * exp(static_cast<double>(s_r[w]) - static_cast<double>(gm));
  }
  const double lse = static_cast<double>(gm) + log(gs);
  // merge the waves' lists: lane j holds entries j and j + 64 of the
  // concatenated lists (entry e = entry e % K of wave e / K), offering the
  // better of the two it still has
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
      cand_lp[row * K + k] = static_cast<float>(static_cast<double>(v) - lse);
    }
  }
}

__device__ __forceinline__ int meta_pack(int depth, int rank, int parent) {
  return ((parent + 1) << 10) | (depth << 5) | rank;
}
__device__ __forceinline__ int meta_depth(int m) { return (m >> 5) & 31; }
__device__ __forceinline__ int meta_rank(int m) { return m & 31; }
__device__ __forceinline__ int meta_parent(int m) { return (m >> 10) - 1; }

// One wave per sequence.  The queue lives in registers, sorted (best score
// first, equal scores by lower slot; a slot is the push counter): entry
// e = 64 r + lane is held by `lane` in register r, with its slot, its
// (depth, rank, parent) and its parent's score.  Only the best N - n entries
// are kept (n = nodes popped so far): insertions only push an entry down, so
// one ranked N - n or lower is never popped.  A round is a few lane-parallel
// steps whatever w is:
//  1. the round's min(w, budget left, queued) candidates are the queue's
//     first entries, in pop order;
//  2. each popped node's successors, its next sibling (depth >= 2) and its
//     first child (below the maximum depth), get slots in pop order (a prefix
//     count over the popped entries);
//  3. the rest of the queue and the new candidates merge: an entry's place is
//     its place in its own group plus the number of entries of the other group
//     that sort before it.  The candidates are visited one at a time (their
//     values read out of their lanes), each compared with every queued entry
//     at once; the merged queue is scattered through LDS and read back.
// The popped nodes are then flattened by depth (stable) and their parents
// renumbered.
__global__ __launch_bounds__(64) void tree_build_kernel(const int32_t* __restrict__ cand_tok,
                                                        const float* __restrict__ cand_lp, int L,
                                                        int K, int N, int w,
                                                        int32_t* __restrict__ tokens,
                                                        int32_t* __restrict__ parent,
                                                        int32_t* __restrict__ depth,
                                                        float* __restrict__ score,
                                                        int32_t* __restrict__ num_nodes) {
  static_assert(TV_MAX_NODES <= 128, "two queue entries per lane");
  __shared__ float s_lp[TV_TREE_MAX_DEPTH * TV_TREE_MAX_TOPK];
  __shared__ float n_score[TV_MAX_NODES];  // popped nodes, in pop order
  __shared__ int n_meta[TV_MAX_NODES];
  __shared__ float x_score[TV_MAX_NODES];  // the merged queue, scattered by place
  __shared__ int x_slot[TV_MAX_NODES];
  __shared__ int x_meta[TV_MAX_NODES];
  __shared__ float x_ps[TV_MAX_NODES];
  __shared__ int s_new[TV_MAX_NODES];
  const int b = blockIdx.x, lane = threadIdx.x;
  const float* lp_b = cand_lp + static_cast<size_t>(b) * L * K;
  for (int e = lane; e < L * K; e += 64) s_lp[e] = lp_b[e];
  __syncthreads();
  // the roots: the K depth-1 candidates in rank order (slots 0 .. K - 1), whose
  // log-probabilities decrease: they are the sorted queue (ties keep rank order)
  int queued = min(K, N);
  float qs[2], qp[2];
  int qsl[2], qm[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int e = 64 * r + lane;
    const float v = s_lp[min(e, L * K - 1)];
    qs[r] = e < queued ? v : -INFINITY;
    qsl[r] = e;
    qm[r] = meta_pack(1, e < K ? e : 0, -1);
    qp[r] = 0.0f;
  }
  int pushed = K;  // slots used
  int n = 0;       // popped nodes
  while (n < N && queued > 0) {
    const int take = min(min(w, N - n), queued);
    const int cap = N - n - take;  // entries worth keeping after this round
    int nc;
    if (take == 1) {
      // one pop (entry 0) and at most two candidates, all wave-uniform: every
      // comparison in one straight-line block
      const float ps = readlane_f(qs[0], 0), pp = readlane_f(qp[0], 0);
      const int pm = __builtin_amdgcn_readlane(qm[0], 0);
      if (lane == 0) {
        n_score[n] = ps;
        n_meta[n] = pm;
      }
      const int d = meta_depth(pm), rk = meta_rank(pm), par = meta_parent(pm);
      const bool sib = (d >= 2) & (rk + 1 < K), child = d < L;
      const float s_sib = pp + s_lp[min(max((d - 1) * K + rk + 1, 0), L * K - 1)];
      const float s_child = ps + s_lp[min(d * K, L * K - 1)];
      const int sl_sib = pushed, sl_child = pushed + static_cast<int>(sib);
      int pos_sib = static_cast<int>(child & cand_before(s_child, sl_child, s_sib, sl_sib));
      int pos_child = static_cast<int>(sib & cand_before(s_sib, sl_sib, s_child, sl_child));
      bool rest[2];
      int below[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e = 64 * r + lane;
        rest[r] = (e >= 1) & (e < queued);
        below[r] = e - 1 + static_cast<int>(sib & cand_before(s_sib, sl_sib, qs[r], qsl[r])) +
                   static_cast<int>(child & cand_before(s_child, sl_child, qs[r], qsl[r]));
        pos_sib += __popcll(__ballot(rest[r] & cand_before(qs[r], qsl[r], s_sib, sl_sib)));
        pos_child += __popcll(__ballot(rest[r] & cand_before(qs[r], qsl[r], s_child, sl_child)));
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (rest[r] & (below[r] < cap)) {
          x_score[below[r]] = qs[r];
          x_slot[below[r]] = qsl[r];
          x_meta[below[r]] = qm[r];
          x_ps[below[r]] = qp[r];
        }
      }
      // lane 0 places the sibling, lane 1 the child
      const bool mine = lane == 0 ? sib & (pos_sib < cap) : (lane == 1) & child & (pos_child < cap);
      if (mine) {
        const int at = lane == 0 ? pos_sib : pos_child;
        x_score[at] = lane == 0 ? s_sib : s_child;
        x_slot[at] = lane == 0 ? sl_sib : sl_child;
        x_meta[at] = lane == 0 ? meta_pack(d, rk + 1, par) : meta_pack(d + 1, 0, n);
        x_ps[at] = lane == 0 ? pp : ps;
      }
      nc = static_cast<int>(sib) + static_cast<int>(child);
    } else {
      // 1, 2. pop entries 0 .. take - 1; their successors, candidate v = 2 r
      // (sibling) or 2 r + 1 (child) of the lane's entry in register r
      float cs[4], cp[4];
      int cm[4], csl[4];
      bool cv[4];
      int base = 0;
  #pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e = 64 * r + lane;
        const bool pop = e < take;
        if (pop) {
          n_score[n + e] = qs[r];
          n_meta[n + e] = qm[r];
        }
        const int d = meta_depth(qm[r]), rk = meta_rank(qm[r]), par = meta_parent(qm[r]);
        const float lp_sib = s_lp[min(max((d - 1) * K + rk + 1, 0), L * K - 1)];
        const float lp_child = s_lp[min(d * K, L * K - 1)];
        cv[2 * r] = pop & (d >= 2) & (rk + 1 < K);
        cv[2 * r + 1] = pop & (d < L);
        cs[2 * r] = qp[r] + lp_sib;
        cm[2 * r] = meta_pack(d, rk + 1, par);
        cp[2 * r] = qp[r];
        cs[2 * r + 1] = qs[r] + lp_child;
        cm[2 * r + 1] = meta_pack(d + 1, 0, n + e);
        cp[2 * r + 1] = qs[r];
        // slots in pop order, the sibling first: an exclusive prefix count of
        // the successors over the lanes (two ballots)
        const int cnt = static_cast<int>(cv[2 * r]) + static_cast<int>(cv[2 * r + 1]);
        const uint64_t b1 = __ballot(cnt >= 1), b2 = __ballot(cnt >= 2);
        const int before =
            static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b1 >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b1), 0u)) +
                             __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b2 >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b2), 0u)));
        csl[2 * r] = pushed + base + before;
        csl[2 * r + 1] = pushed + base + before + static_cast<int>(cv[2 * r]);
        base += __popcll(b1) + __popcll(b2);
      }
      nc = base;
      // 3. merge, lane-parallel: each lane ranks its own queued entries and
      // candidates against the other group, whose members are read out one
      // at a time.  A queued entry e >= take keeps its order among the rest
      // and moves down by the candidates that sort before it; a candidate's
      // place is the queued entries and the candidates before it.
      bool rest[2];
      int below[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int e = 64 * r + lane;
        rest[r] = (e >= take) & (e < queued);
        below[r] = e - take;
      }
      int pos[4] = {0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int nsrc = v < 2 ? min(take, 64) : take - 64;  // the popped lanes of register v / 2
        for (int src = 0; src < nsrc; ++src) {
          if (__builtin_amdgcn_readlane(static_cast<int>(cv[v]), src) == 0) continue;
          const float c_s = readlane_f(cs[v], src);
          const int c_sl = __builtin_amdgcn_readlane(csl[v], src);
#pragma unroll
          for (int r = 0; r < 2; ++r) below[r] += static_cast<int>(cand_before(c_s, c_sl, qs[r], qsl[r]));
#pragma unroll
          for (int u = 0; u < 4; ++u) pos[u] += static_cast<int>(cand_before(c_s, c_sl, cs[u], csl[u]));
        }
      }
      for (int j = take; j < queued; ++j) {
        const float q0 = readlane_f(qs[0], j & 63), q1 = readlane_f(qs[1], j & 63);
        const int l0 = __builtin_amdgcn_readlane(qsl[0], j & 63), l1 = __builtin_amdgcn_readlane(qsl[1], j & 63);
        const float q_s = j < 64 ? q0 : q1;
        const int q_sl = j < 64 ? l0 : l1;
#pragma unroll
        for (int u = 0; u < 4; ++u) pos[u] += static_cast<int>(cand_before(q_s, q_sl, cs[u], csl[u]));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (cv[u] & (pos[u] < cap)) {
          x_score[pos[u]] = cs[u];
          x_slot[pos[u]] = csl[u];
          x_meta[pos[u]] = cm[u];
          x_ps[pos[u]] = cp[u];
        }
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (rest[r] & (below[r] < cap)) {
          x_score[below[r]] = qs[r];
          x_slot[below[r]] = qsl[r];
          x_meta[below[r]] = qm[r];
          x_ps[below[r]] = qp[r];
        }
      }
    }
    queued = min(queued - take + nc, cap);
    pushed += nc;
    n += take;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = 64 * r + lane;
      const int i = min(e, TV_MAX_NODES - 1);
      const float v = x_score[i];
      const int sl = x_slot[i], m = x_meta[i];
      const float ps = x_ps[i];
      const bool ok = e < queued;
      qs[r] = ok ? v : -INFINITY;
      qsl[r] = ok ? sl : 0x7fffffff;
      qm[r] = ok ? m : meta_pack(1, 0, -1);
      qp[r] = ok ? ps : 0.0f;
    }
    __syncthreads();
  }

  // flatten by depth, stable: new index = nodes of smaller depth + nodes of
  // the same depth popped earlier.  Lane l holds nodes l and l + 64; one
  // ballot per (depth, half) counts them.
  {
    const int d0 = lane < n ? meta_depth(n_meta[lane]) : 0;
    const int d1 = lane + 64 < n ? meta_depth(n_meta[lane + 64]) : 0;
    int before = 0, p0 = 0, p1 = 0;
    for (int d = 1; d <= L; ++d) {
      const uint64_t b0 = __ballot(d0 == d), b1 = __ballot(d1 == d);
      const uint32_t below0 = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b0 >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b0), 0u));
      const uint32_t below1 = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b1 >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b1), 0u));
      if (d0 == d) p0 = before + static_cast<int>(below0);
      if (d1 == d) p1 = before + __popcll(b0) + static_cast<int>(below1);
      before += __popcll(b0) + __popcll(b1);
    }
    if (lane < n) s_new[lane] = p0;
    if (lane + 64 < n) s_new[lane + 64] = p1;
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
