// Streaming-read probe for the benchmark: the HBM read rate a plain kernel
// reaches on this device, printed beside the vendor's 8 TB/s.  Not part of the
// tree-verification library; built into its own shared object.
//
// Each lane reads 16-byte pieces in a grid-stride loop, eight loads in flight,
// and folds them into one word; a workgroup stores its word only when it
// equals a value the data never produces, so the loads cannot be dropped and
// almost nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `src` with `grid`
// workgroups of 256 threads on `stream`; `sink` holds `grid` uint32 words.
// Returns 0 on success, -1 on bad arguments, else the HIP error code.
int tv_probe_stream_read(const void* src, size_t bytes, void* sink, int grid, void* stream) {
  if (src == nullptr || sink == nullptr || grid < 1 || (bytes & 15u) ||
      (reinterpret_cast<uintptr_t>(src) & 15u))
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src), bytes / 16,
                     static_cast<uint32_t*>(sink));
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
