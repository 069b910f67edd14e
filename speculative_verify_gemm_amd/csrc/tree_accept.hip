// Greedy acceptance of a verified draft tree on gfx950, in one launch.
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com).  Section "Producing several tokens from one model
// pass": the main model checks all drafted positions in one pass, keeps the
// valid prefix and goes on from the first rejected position with its own
// token (five drafted, the first four agreed: the sequence advances by five).
// Section "Issue with parallel draft generation": with a tree of drafts the
// main model accepts the longest valid path.  The readings (include/svgemm.h,
// tree_accept_greedy): node 0 is the root, parent[i] < i; the target's choice
// at a node is the first largest logit of its row; a node is valid when its
// parent is valid and its token is the parent's choice; the deepest valid node
// wins, the smaller index among equal depths; the pass emits the path's tokens
// and the choice at its end.
//
// Work: the logits (T rows of V fp32, the only bulk data) stream once from HBM.
//  1. Every workgroup reduces one slice of one row to the 64-bit key
//     (order-preserving bits of the value) << 32 | (2^32 - 1 - index), so that
//     the largest key is the largest value and, among equal values, the
//     smallest index; it folds the key into its row's slot of the workspace
//     with a 64-bit atomic max, then counts itself in with an atomic add.
//  2. The workgroup whose count completes the grid reads the row keys (every
//     other workgroup has folded its key before counting itself: release and
//     acquire order at device scope), clears the workspace for the next call,
//     and walks the tree (at most 32 nodes, one thread: nodes only depend on
//     earlier nodes).
// Nothing waits for another workgroup, so no launch order or residency is
// assumed.
#include <algorithm>

#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxNodes = 32;
constexpr int kUnroll = 8;  // float4 loads in flight per thread

typedef unsigned long long u64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Monotone map of fp32 to u32 (larger value -> larger code; -0 < +0).
SVG_DEV u32 order_bits(float v) {
  const u32 b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
SVG_DEV u64 make_key(float v, u32 idx) { return ((u64)order_bits(v) << 32) | (u64)(0xFFFFFFFFu - idx); }
SVG_DEV u64 umax64(u64 a, u64 b) { return a > b ? a : b; }

SVG_DEV u64 shfl_xor64(u64 v, int m) {
  const int lo = __shfl_xor((int)(u32)v, m), hi = __shfl_xor((int)(u32)(v >> 32), m);
  return ((u64)(u32)hi << 32) | (u64)(u32)lo;
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads) void k_tree_accept(const float* __restrict__ logits, int T, int V, int S,
                                                         int L, const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ draft, int32_t* target,
                                                         int32_t* path, int32_t* emit, int32_t* n_emit,
                                                         u64* keys, u32* arrivals) {
  __shared__ u64 wave_best[kThreads / 64];
  __shared__ int last;
  __shared__ int par[kMaxNodes], tok[kMaxNodes], tgt[kMaxNodes], route[kMaxNodes], depth[kMaxNodes];
  __shared__ int best_node, depth_best, bad;

  // ---- 1. slice maximum
  const int row = blockIdx.x / S, s = blockIdx.x % S;
  const int lo = s * L, hi = min(V, lo + L);
  const float* r = logits + (size_t)row * (size_t)V;
  u64 best = 0;  // below every key of a non-NaN value
  if constexpr (VEC4) {  // lo and V are multiples of 4; the row start is 16-byte aligned
    const f32x4* r4 = reinterpret_cast<const f32x4*>(r);
    const int c0 = lo >> 2, c1 = hi >> 2;
    for (int c = c0 + threadIdx.x; c < c1; c += kThreads * kUnroll) {
      f32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int cu = c + u * kThreads;
        if (cu < c1) v[u] = __builtin_nontemporal_load(r4 + cu);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int cu = c + u * kThreads;
        if (cu < c1) {
          const u32 k0 = 4u * (u32)cu;
          best = umax64(best, make_key(v[u][0], k0));
          best = umax64(best, make_key(v[u][1], k0 + 1));
          best = umax64(best, make_key(v[u][2], k0 + 2));
          best = umax64(best, make_key(v[u][3], k0 + 3));
        }
      }
    }
  } else {
    for (int k = lo + threadIdx.x; k < hi; k += kThreads) best = umax64(best, make_key(r[k], (u32)k));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor64(best, m));
  if ((threadIdx.x & 63) == 0) wave_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    u64 b = wave_best[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = umax64(b, wave_best[w]);
    __hip_atomic_fetch_max(keys + row, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // release: the key above is folded before the count; acquire: the last
    // workgroup sees every key folded before the counts it read
    const u32 before = __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = before == gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;

  // ---- 2. the last workgroup: choices, reset, tree walk
  const int t = threadIdx.x;
  if (t < T) {
    const u64 key = __hip_atomic_load(keys + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int c = (int)(0xFFFFFFFFu - (u32)key);
    target[t] = c;
    tgt[t] = c;
    par[t] = parent[t];
    tok[t] = draft[t];
    __hip_atomic_store(keys + t, (u64)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (t == 0) __hip_atomic_store(arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (t == 0) {
    int b = par[0] != -1;
    for (int i = 1; i < T; ++i) b |= !(par[i] >= 0 && par[i] < i);
    bad = b;
    if (!b) {
      // valid[i] / depth[i] only depend on the parent, an earlier node
      unsigned valid = 1u;  // bit i: node i valid (T <= 32)
      depth[0] = 0;
      int bn = 0, bd = 0;
      for (int i = 1; i < T; ++i) {
        const int p = par[i];
        depth[i] = depth[p] + 1;
        if (((valid >> p) & 1u) && tok[i] == tgt[p]) {
          valid |= 1u << i;
          if (depth[i] > bd) { bn = i; bd = depth[i]; }
        }
      }
      for (int k = bd - 1, n = bn; k >= 0; --k, n = par[n]) route[k] = n;
      best_node = bn;
      depth_best = bd;
    }
  }
  __syncthreads();
  if (t < T) {
    if (bad) {
      path[t] = -1;
      emit[t] = -1;
    } else {
      const int d = depth_best;
      path[t] = t < d ? route[t] : -1;
      emit[t] = t < d ? tok[route[t]] : (t == d ? tgt[best_node] : -1);
    }
  }
  if (t == 0) *n_emit = bad ? -1 : depth_best + 1;
}

}  // namespace

hipError_t svg_launch_tree_accept(const float* logits, int T, int V, const int32_t* parent, const int32_t* draft,
                                  int32_t* target, int32_t* path, int32_t* emit, int32_t* n_emit, void* workspace,
                                  hipStream_t stream) {
  // slices per row: about 8192 values each, and no more than two workgroups
  // per CU over the whole grid
  const int by_size = (V + 8191) / 8192;
  const int by_grid = std::max(1, 2 * svg_cu_count() / T);
  const int S = std::max(1, std::min(by_size, by_grid));
  const int L = ((V + S - 1) / S + 3) / 4 * 4;  // values per slice, a multiple of 4
  u64* keys = static_cast<u64*>(workspace);
  u32* arrivals = reinterpret_cast<u32*>(static_cast<char*>(workspace) + 256);
  const bool vec4 = V % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  if (vec4)
    hipLaunchKernelGGL(k_tree_accept<true>, dim3(T * S), dim3(kThreads), 0, stream, logits, T, V, S, L, parent,
                       draft, target, path, emit, n_emit, keys, arrivals);
  else
    hipLaunchKernelGGL(k_tree_accept<false>, dim3(T * S), dim3(kThreads), 0, stream, logits, T, V, S, L, parent,
                       draft, target, path, emit, n_emit, keys, arrivals);
  return hipGetLastError();
}
