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
// LDS in tiles of 32: K row-major, V row-major, both padded by 16 bytes per
// row to spread LDS banks; the next tile's global loads are in flight while
// the current one is computed.  Scores are formed transposed (S^T = K Q^T) so
// that each lane's MFMA result holds keys of a single query row: the online
// softmax then needs only two cross-lane steps per row, and the probabilities
// feed the P.V MFMA (O^T = V^T P^T) straight from registers.  The split that
// holds the end of the context also takes the node keys, masked by the
// ancestor word of each row's node.  A split writes fp32 partials (acc, m, l);
// a second kernel merges them by log-sum-exp.  A sequence whose keys fit one
// split writes its output directly.
#include "tv_internal.h"

namespace tv {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = kWaves * 16;  // query rows per workgroup
constexpr int kTile = 32;           // keys per LDS tile
constexpr int kThreads = kWaves * 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int D>
struct Cfg {
  static constexpr int kEsz = sizeof(T);
  static constexpr int kRowBytes = D * kEsz;
  static constexpr int kPitch = kRowBytes + 16;  // LDS row pitch in bytes
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kChunksPerThread = kTile * kChunksPerRow / kThreads;
  static constexpr int kDT = D / 16;  // 16-wide output column tiles
  static_assert(kTile * kChunksPerRow % kThreads == 0, "tile must split evenly over threads");
};

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

// smallest position id of the tree (N <= 64 nodes, read by wave 0)
__device__ __forceinline__ int tree_min_pos(const int32_t* pos_b, int N, int* s_min) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    int v = tid < N ? pos_b[tid] : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
    if (tid == 0) *s_min = v;
  }
  __syncthreads();
  return *s_min;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, typename TO, int D>
__global__ __launch_bounds__(kThreads, 2) void attn_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kn, const T* __restrict__ vn,
    const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ bt,
    int max_blocks, int num_blocks, const int32_t* __restrict__ ctx_len, int max_ctx,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ pos, int N, int Hq, int Hkv,
    int G, int rows, int row_groups, int nsplit_max, int split_tokens, int window,
    float scale_log2, int total_units, TO* __restrict__ out, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml) {
  using C = Cfg<T, D>;
  __shared__ __align__(16) unsigned char Ks[kTile * C::kPitch];
  __shared__ __align__(16) unsigned char Vs[kTile * C::kPitch];
  __shared__ int s_pos[64];
  __shared__ int s_min;

  // blocks are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of work units so that row groups sharing a KV stream
  // share an L2
  const int nwg = gridDim.x;
  const int logical = (blockIdx.x % 8) * (nwg / 8) + (blockIdx.x / 8);
  if (logical >= total_units) return;
  const int rg = logical % row_groups;
  int rest = logical / row_groups;
  const int s = rest % nsplit_max;
  rest /= nsplit_max;
  const int g = rest % Hkv;
  const int b = rest / Hkv;

  const int tid = threadIdx.x;
  const int32_t* pos_b = pos + static_cast<size_t>(b) * N;
  if (tid < 64) s_pos[tid] = tid < N ? pos_b[tid] : 0;
  const int min_pos = tree_min_pos(pos_b, N, &s_min);
  const SeqPlan sp = seq_plan(ctx_len[b], max_ctx, window, min_pos, nsplit_max, split_tokens);
  if (s >= sp.nsplit) return;  // uniform over the workgroup
  const int k0 = sp.start + s * sp.split_len;
  const int k1 = min(k0 + sp.split_len, sp.end);
  const bool last = s == sp.nsplit - 1;
  const int nctx_tiles = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;
  const int ntiles = nctx_tiles + (last ? (N + kTile - 1) / kTile : 0);

  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int R = rg * kRows + wave * 16 + lr;
  const bool row_ok = R < rows;
  const int t = row_ok ? R / G : 0;
  const int hl = row_ok ? R % G : 0;
  const int row_pos = pos_b[t];
  const uint64_t row_anc = anc[static_cast<size_t>(b) * N + t];
  const size_t qoff = ((static_cast<size_t>(b) * N + t) * Hq + g * G + hl) * D;

  // query fragments (MFMA B operand): row lr, 8 (bf16) or 1 (fp32) dims per k step
  constexpr int kQ = (sizeof(T) == 2) ? D / 32 : D / 4;
  bf16x8_t qf_b[sizeof(T) == 2 ? kQ : 1];
  float qf_f[sizeof(T) == 4 ? kQ : 1];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(q + qoff + ks * 32 + lg * 8)
                       : make_uint4(0, 0, 0, 0);
      qf_b[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) qf_f[ks] = row_ok ? q[qoff + ks * 4 + lg] : 0.0f;
  }

  f32x4_t acc[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  const int32_t* bt_b = bt + static_cast<size_t>(b) * max_blocks;
  const unsigned char* kcb = reinterpret_cast<const unsigned char*>(kc);
  const unsigned char* vcb = reinterpret_cast<const unsigned char*>(vc);
  const unsigned char* knb = reinterpret_cast<const unsigned char*>(kn);
  const unsigned char* vnb = reinterpret_cast<const unsigned char*>(vn);

  uint4 rk[C::kChunksPerThread], rv[C::kChunksPerThread];
  auto load_tile = [&](int it) {
    const bool is_node = it >= nctx_tiles;
    const int base = is_node ? (it - nctx_tiles) * kTile : k0 + it * kTile;
    const int lim = is_node ? N : k1;
#pragma unroll
    for (int c = 0; c < C::kChunksPerThread; ++c) {
      const int chunk = tid + c * kThreads;
      const int j = chunk / C::kChunksPerRow;
      const int part = chunk % C::kChunksPerRow;
      const int key = base + j;
      if (key < lim) {
        size_t off;
        const unsigned char *ksrc, *vsrc;
        if (is_node) {
          off = ((static_cast<size_t>(b) * N + key) * Hkv + g) * C::kRowBytes + part * 16;
          ksrc = knb;
          vsrc = vnb;
        } else {
          int page = bt_b[key >> 4];
          page = min(max(page, 0), num_blocks - 1);
          off = ((static_cast<size_t>(page) * Hkv + g) * 16 + (key & 15)) * C::kRowBytes + part * 16;
          ksrc = kcb;
          vsrc = vcb;
        }
        rk[c] = *reinterpret_cast<const uint4*>(ksrc + off);
        rv[c] = *reinterpret_cast<const uint4*>(vsrc + off);
      } else {
        rk[c] = make_uint4(0, 0, 0, 0);
        rv[c] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < C::kChunksPerThread; ++c) {
      const int chunk = tid + c * kThreads;
      const int j = chunk / C::kChunksPerRow;
      const int part = chunk % C::kChunksPerRow;
      *reinterpret_cast<uint4*>(Ks + j * C::kPitch + part * 16) = rk[c];
      *reinterpret_cast<uint4*>(Vs + j * C::kPitch + part * 16) = rv[c];
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (it + 1 < ntiles) load_tile(it + 1);

    const bool is_node = it >= nctx_tiles;
    const int base = is_node ? (it - nctx_tiles) * kTile : k0 + it * kTile;
    const int lim = is_node ? N : k1;

    // S^T for two 16-key halves: lane holds keys 16j + 4lg + i of row lr
    f32x4_t S[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      S[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const unsigned char* krow = Ks + (16 * j + lr) * C::kPitch;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int ks = 0; ks < kQ; ++ks) {
          bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(krow + ks * 64 + lg * 16));
          S[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf_b[ks], S[j], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < kQ; ++ks) {
          float a = *reinterpret_cast<const float*>(krow + (ks * 4 + lg) * 4);
          S[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf_f[ks], S[j], 0, 0, 0);
        }
      }
    }

    // mask, scale into the log2 domain, row max
    float x[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = base + 16 * j + 4 * lg + i;
        bool vis = row_ok && key < lim;
        if (is_node) {
          vis = vis && ((row_anc >> (key & 63)) & 1ull);
          if (window > 0) {
            const int dpos = row_pos - s_pos[key & 63];
            vis = vis && dpos >= 0 && dpos < window;
          }
        } else if (window > 0) {
          const int dpos = row_pos - key;
          vis = vis && dpos >= 0 && dpos < window;
        }
        x[j][i] = vis ? S[j][i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[j][i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    float p[2][4];
    float alpha = 1.0f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[j][i] = 0.0f;
    } else {
      alpha = fast_exp2(m_run - m_new);
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[j][i] = fast_exp2(x[j][i] - m_new);
          ps += p[j][i];
        }
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) acc[dt] *= alpha;
    }

    // O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
      s16x8_t pb16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb16[i] = static_cast<short>(f32_to_bf16(p[0][i]));
        pb16[4 + i] = static_cast<short>(f32_to_bf16(p[1][i]));
      }
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pb16);
      const uint16_t* V16 = reinterpret_cast<const uint16_t*>(Vs);
      constexpr int P16 = C::kPitch / 2;
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
        s16x8_t av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[i] = static_cast<short>(V16[(4 * lg + i) * P16 + dt * 16 + lr]);
          av[4 + i] = static_cast<short>(V16[(16 + 4 * lg + i) * P16 + dt * 16 + lr]);
        }
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), pb,
                                                          acc[dt], 0, 0, 0);
      }
    } else {
      const float* VF = reinterpret_cast<const float*>(Vs);
      constexpr int PF = C::kPitch / 4;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int krow = 16 * j + 4 * lg + i;
#pragma unroll
          for (int dt = 0; dt < C::kDT; ++dt)
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(VF[krow * PF + dt * 16 + lr], p[j][i],
                                                           acc[dt], 0, 0, 0);
        }
    }
  }

  // row sum over the four lanes that share the row
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot = l_tot + __shfl_xor(l_tot, 32, 64);
  if (!row_ok) return;

  if (sp.nsplit == 1) {
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
    const size_t ub = ((static_cast<size_t>(b) * Hkv + g) * nsplit_max + s) * rows + R;
    float* pa = ws_acc + ub * D;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt)
      *reinterpret_cast<float4*>(pa + dt * 16 + 4 * lg) =
          make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (lg == 0) ws_ml[ub] = make_float2(m_run, l_tot);
  }
}

// Log-sum-exp merge of the split partials of sequences that used more than
// one split.  Thread = 4 consecutive output columns of one row.
template <typename TO, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(
    const int32_t* __restrict__ ctx_len, int max_ctx, const int32_t* __restrict__ pos, int N,
    int Hq, int Hkv, int G, int rows, int nsplit_max, int split_tokens, int window,
    const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml, TO* __restrict__ out) {
  constexpr int kTpr = D / 4;              // threads per row
  constexpr int kRpb = 256 / kTpr;         // rows per block
  __shared__ int s_min;
  const int chunks = (rows + kRpb - 1) / kRpb;
  const int bg = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int g = bg % Hkv;
  const int b = bg / Hkv;
  const int32_t* pos_b = pos + static_cast<size_t>(b) * N;
  const int min_pos = tree_min_pos(pos_b, N, &s_min);
  const SeqPlan sp = seq_plan(ctx_len[b], max_ctx, window, min_pos, nsplit_max, split_tokens);
  if (sp.nsplit == 1) return;
  const int R = chunk * kRpb + threadIdx.x / kTpr;
  if (R >= rows) return;
  const int d0 = (threadIdx.x % kTpr) * 4;
  const size_t ub0 = (static_cast<size_t>(b) * Hkv + g) * nsplit_max * rows + R;
  float mx = -INFINITY;
  for (int s = 0; s < sp.nsplit; ++s) mx = fmaxf(mx, ws_ml[ub0 + static_cast<size_t>(s) * rows].x);
  float L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < sp.nsplit; ++s) {
    const size_t ub = ub0 + static_cast<size_t>(s) * rows;
    const float2 ml = ws_ml[ub];
    const float w = ml.x == -INFINITY ? 0.0f : fast_exp2(ml.x - mx);
    L += w * ml.y;
    const float4 a = *reinterpret_cast<const float4*>(ws_acc + ub * D + d0);
    o.x += w * a.x;
    o.y += w * a.y;
    o.z += w * a.z;
    o.w += w * a.w;
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
  const long long units = static_cast<long long>(B) * Hkv * pl.nsplit * pl.row_groups;
  const long long grid = (units + 7) / 8 * 8;
  float* ws_acc = nullptr;
  float2* ws_ml = nullptr;
  if (pl.nsplit > 1) {
    ws_acc = static_cast<float*>(ws);
    ws_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                      static_cast<size_t>(B) * Hkv * pl.nsplit * pl.rows * D * 4);
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_split_kernel<T, TO, D>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k_node),
                     static_cast<const T*>(v_node), static_cast<const T*>(k_cache),
                     static_cast<const T*>(v_cache), block_table, max_blocks, num_blocks, ctx_len,
                     max_ctx, anc, pos, N, Hq, Hkv, pl.G, pl.rows, pl.row_groups, pl.nsplit,
                     pl.split_tokens, window, scale_log2, static_cast<int>(units),
                     static_cast<TO*>(out), ws_acc, ws_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  constexpr int kRpb = 256 / (D / 4);
  const unsigned mgrid = static_cast<unsigned>(B) * Hkv * ((pl.rows + kRpb - 1) / kRpb);
  hipLaunchKernelGGL((attn_merge_kernel<TO, D>), dim3(mgrid), dim3(256), 0, stream, ctx_len, max_ctx,
                     pos, N, Hq, Hkv, pl.G, pl.rows, pl.nsplit, pl.split_tokens, window, ws_acc,
                     ws_ml, static_cast<TO*>(out));
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int B, int N, int Hq, int Hkv, int D, int max_ctx_len, int window) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.rows = p.G * N;
  p.row_groups = (p.rows + kRows - 1) / kRows;
  const int range = window > 0 ? (max_ctx_len < window ? max_ctx_len : window) : max_ctx_len;
  // aim for a few thousand workgroups, but keep each split long enough that
  // its fp32 partials stay small next to the keys it streams
  const long long units = static_cast<long long>(B) * Hkv * p.row_groups;
  long long want = (4096 + units - 1) / units;
  const int min_split = 1024;
  long long cap = (range + min_split - 1) / min_split;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  int st = static_cast<int>((range + want - 1) / want);
  st = (st + kTile - 1) / kTile * kTile;
  if (st < kTile) st = kTile;
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
#define TV_ATTN_DIMS(TYPE, OTYPE)            \
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
