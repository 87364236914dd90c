// Greedy tree walk with the bonus token.
//
// Serve-integration spec, sections "What's proven" and "3. Rejection
// sampler: tree walk": from the root follow the child whose token equals the
// target argmax at the current node, then emit the argmax where no child
// matches.  Two kernels: a row argmax over the vocabulary (an HBM stream, one
// workgroup per logits row), then one wave per tree that walks the parent
// pointers (lanes = nodes; ballots find the matching child each step).
#include <atomic>

#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kArgmaxThreads = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

struct Best {
  float v;
  int i;
};

// larger value wins; on equal values the lower index wins
__device__ __forceinline__ Best better(Best a, Best b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ Best wave_best(Best x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Best y;
    y.v = __shfl_xor(x.v, off, 64);
    y.i = __shfl_xor(x.i, off, 64);
    x = better(x, y);
  }
  return x;
}

__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void scan_chunk(const u32x4_t& c, int first, Best& best) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float lo = __uint_as_float(w[k] << 16);
      float hi = __uint_as_float(w[k] & 0xffff0000u);
      if (lo > best.v) { best.v = lo; best.i = first + 2 * k; }
      if (hi > best.v) { best.v = hi; best.i = first + 2 * k + 1; }
    }
  } else {
    const float f[4] = {__uint_as_float(c[0]), __uint_as_float(c[1]), __uint_as_float(c[2]),
                        __uint_as_float(c[3])};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (f[k] > best.v) { best.v = f[k]; best.i = first + k; }
  }
}

// am[row] = argmax_v logits[row, v]; rows are V elements long.
template <typename T>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const T* __restrict__ logits,
                                                                int V, int32_t* __restrict__ am) {
  const size_t row = blockIdx.x;
  const T* p = logits + row * static_cast<size_t>(V);
  const int tid = threadIdx.x;
  // strict '>' while a thread scans increasing indices keeps its first maximum;
  // the start value lets the first element (even -inf) win
  Best best{-INFINITY, 0x7fffffff};
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  const bool vec = ((static_cast<size_t>(V) * sizeof(T)) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  if (vec) {
    const u32x4_t* pc = reinterpret_cast<const u32x4_t*>(p);
    const int nchunk = V / E;
    int c = tid;
    for (; c + (kUnroll - 1) * kArgmaxThreads < nchunk; c += kUnroll * kArgmaxThreads) {
      u32x4_t r[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) r[u] = __builtin_nontemporal_load(pc + c + u * kArgmaxThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        Best cand{-INFINITY, 0x7fffffff};
        scan_chunk<T>(r[u], (c + u * kArgmaxThreads) * E, cand);
        best = better(best, cand);
      }
    }
    for (; c < nchunk; c += kArgmaxThreads) {
      Best cand{-INFINITY, 0x7fffffff};
      scan_chunk<T>(pc[c], c * E, cand);
      best = better(best, cand);
    }
  } else {
    for (int v = tid; v < V; v += kArgmaxThreads) {
      Best cand{load_elem(p, v), v};
      best = better(best, cand);
    }
  }
  // an all -inf chunk leaves its candidate index at the sentinel; -inf rows
  // are outside the contract, so any in-range index is acceptable there
  best = wave_best(best);
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  const int w = tid / 64;
  if ((tid & 63) == 0) { sv[w] = best.v; si[w] = best.i; }
  __syncthreads();
  if (tid == 0) {
    Best r{sv[0], si[0]};
    for (int k = 1; k < kArgmaxThreads / 64; ++k) r = better(r, Best{sv[k], si[k]});
    if (r.i < 0 || r.i >= V) r.i = 0;
    am[row] = r.i;
  }
}

// Lane l holds nodes l and l + 64 (trees of up to 128 nodes): one ballot per
// half finds the matching children, the lower half first, so the lowest
// matching index wins.
constexpr int kWalkSlots = (TV_MAX_NODES + 63) / 64;

__global__ __launch_bounds__(64) void walk_kernel(const int32_t* __restrict__ tokens,
                                                  const int32_t* __restrict__ parent,
                                                  const int32_t* __restrict__ am, int N,
                                                  int32_t* __restrict__ acc_tok,
                                                  int32_t* __restrict__ acc_node,
                                                  int32_t* __restrict__ num_acc) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const size_t base = static_cast<size_t>(b) * N;
  const int32_t* amb = am + static_cast<size_t>(b) * (N + 1);
  int tok[kWalkSlots], par[kWalkSlots];
  bool valid[kWalkSlots];
#pragma unroll
  for (int s = 0; s < kWalkSlots; ++s) {
    const int n = t + 64 * s;
    const bool act = n < N;
    tok[s] = act ? tokens[base + n] : -1;
    par[s] = act ? parent[base + n] : -2;
    valid[s] = act && par[s] >= -1 && par[s] < n;
  }

  int cur = -1, a = 0;
  int my_node[kWalkSlots], my_tok[kWalkSlots];
#pragma unroll
  for (int s = 0; s < kWalkSlots; ++s) my_node[s] = my_tok[s] = -1;
  int pred = amb[0];
  // a matched child always has a larger index than its parent, so the walk
  // ends within N steps
  for (int step = 0; step < N; ++step) {
    int i = -1;
#pragma unroll
    for (int s = 0; s < kWalkSlots; ++s) {
      const uint64_t m = __ballot(valid[s] && par[s] == cur && tok[s] == pred);
      if (i < 0 && m != 0ull) i = 64 * s + __ffsll(static_cast<unsigned long long>(m)) - 1;
    }
    if (i < 0) break;
    // accepted entry a lives in lane a % 64, slot a / 64
#pragma unroll
    for (int s = 0; s < kWalkSlots; ++s)
      if (t + 64 * s == a) { my_node[s] = i; my_tok[s] = pred; }
    ++a;
    cur = i;
    pred = amb[1 + i];
  }
  // pred is now the bonus token (argmax at the last accepted node)
  int32_t* ot = acc_tok + static_cast<size_t>(b) * (N + 1);
#pragma unroll
  for (int s = 0; s < kWalkSlots; ++s) {
    const int n = t + 64 * s;
    if (n < N) acc_node[base + n] = n < a ? my_node[s] : -1;
    if (n < N + 1) ot[n] = n < a ? my_tok[s] : (n == a ? pred : -1);
  }
  // slot N of the token row when the lane slots end before it (never below a)
  if (t == 0 && N == 64 * kWalkSlots) ot[N] = (N == a) ? pred : -1;
  if (t == 0) num_acc[b] = a;
}

}  // namespace

namespace {

// Argmax scratch of the allocation-free walk: one int32 per logits row.  Each
// GPU holds its own copy until the process ends.  Host code never passes this
// name to a kernel (on the host it is a stand-in, not a device address); it
// uses the per-device address from hipGetSymbolAddress below.
static __device__ __align__(256) int32_t scratch[TV_WALK_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::atomic<int32_t*> scratch_ptr[kMaxDevices];  // device address per device id

// The device address of this device's scratch, looked up once per device
// (with that device current) and kept.
hipError_t scratch_address(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    int32_t* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return hipSuccess;
    }
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  if (cached) scratch_ptr[dev].store(static_cast<int32_t*>(ptr), std::memory_order_release);
  *out = static_cast<int32_t*>(ptr);
  return hipSuccess;
}

}  // namespace

hipError_t launch_walk(const int32_t* tokens, const int32_t* parent, const void* logits, int B,
                       int N, int V, tv_dtype dtype, int32_t* acc_tok, int32_t* acc_node,
                       int32_t* num_acc, int32_t* argmax_ws, hipStream_t stream) {
  const unsigned rows = static_cast<unsigned>(B) * static_cast<unsigned>(N + 1);
  if (dtype == TV_BF16)
    hipLaunchKernelGGL(argmax_kernel<uint16_t>, dim3(rows), dim3(kArgmaxThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), V, argmax_ws);
  else
    hipLaunchKernelGGL(argmax_kernel<float>, dim3(rows), dim3(kArgmaxThreads), 0, stream,
                       static_cast<const float*>(logits), V, argmax_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk_kernel, dim3(B), dim3(64), 0, stream, tokens, parent, argmax_ws, N,
                     acc_tok, acc_node, num_acc);
  return hipGetLastError();
}

// The walk with the static scratch: every row's argmax is written before the
// walk reads it, so the array's earlier contents do not matter.  The caller
// has checked B * (N + 1) <= TV_WALK_NOALLOC_MAX_ROWS.
hipError_t launch_walk_noalloc(const int32_t* tokens, const int32_t* parent, const void* logits,
                               int B, int N, int V, tv_dtype dtype, int32_t* acc_tok,
                               int32_t* acc_node, int32_t* num_acc, hipStream_t stream) {
  int32_t* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_walk(tokens, parent, logits, B, N, V, dtype, acc_tok, acc_node, num_acc, ws, stream);
}

}  // namespace tv
