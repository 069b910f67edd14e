// Greedy acceptance of a verified draft tree on gfx950, in one launch.
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com).  Section "Producing several tokens from one model
// pass": the main model checks all drafted positions in one pass, keeps the
// valid prefix and goes on from the first rejected position with its own
// token (five drafted, the first four agreed: the sequence advances by five).
// Section "Issue with parallel draft generation": over a tree of drafts,
// the deepest root path that agrees at every edge is kept.  The readings (include/svgemm.h,
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
//     with a 64-bit atomic max, then -- with an operand that depends on the
//     max's returned value -- counts itself in its row (the workgroup
//     completing a row counts the row in).
//  2. The workgroup completing the last row reads the row keys (every
//     workgroup's key was acknowledged before it counted itself), clears the
//     workspace for the next call, and walks the tree with one lane per node
//     (at most 32): pointer jumping over the parent links gives every node's
//     depth and whether its whole root path agrees.
// Nothing waits for another workgroup, so no launch order or residency is
// assumed.
#include <algorithm>
#include <mutex>

#include "../../include/svgemm.h"
#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxNodes = 32;  // one lane per node in the walk, bit room in its sort key
static_assert(kMaxNodes <= 64 && kMaxNodes <= 255, "nodes must fit a wave and the 8-bit index field");
constexpr int kUnroll = 8;  // float4 loads in flight per thread

typedef unsigned long long u64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Monotone map of fp32 to u32 (larger value -> larger code).  -0 and +0 are
// one value (equal maxima go to the smaller index), so -0 takes +0's code:
// -0 + 0 = +0 when rounding to nearest.
SVG_DEV u32 order_bits(float v) {
  const u32 b = __float_as_uint(v + 0.0f);
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
                                                         u64* keys, u32* row_count, u32* rows_done) {
  __shared__ u64 wave_best[kThreads / 64];
  __shared__ int last;
  // every argument in one round trip (else the slice bounds wait for S and L
  // before the rest is requested)
  asm volatile("" ::"s"(logits), "s"(T), "s"(V), "s"(S), "s"(L), "s"(parent), "s"(draft), "s"(target), "s"(path),
               "s"(emit), "s"(n_emit), "s"(keys), "s"(row_count), "s"(rows_done));

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
    const u64 old = __hip_atomic_fetch_max(keys + row, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The key is performed at the device's coherence point before this
    // workgroup counts itself: the count's operand depends on the value the
    // max returned (an opaque zero made from it), so neither the compiler nor
    // the hardware can issue the count before the max has been performed --
    // no cache-wide write-back is needed, nothing else was written.  The
    // count goes to the row first, and only the workgroup completing a row
    // counts the row in, so no single word takes every workgroup's atomic.
    u32 after_key = (u32)old;
    asm volatile("v_mov_b32 %0, 0" : "=v"(after_key) : "0"(after_key));
    int done = 0;
    if (__hip_atomic_fetch_add(row_count + row, 1u + after_key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        (u32)S - 1)
      done = __hip_atomic_fetch_add(rows_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (u32)T - 1;
    last = done;
  }
  __syncthreads();
  if (!last) return;

  // ---- 2. the last workgroup, one wave, lane i = node i: choices, reset,
  // tree walk.  Its loads are issued after the counts it read returned, and
  // device-scope atomic loads bypass the XCD's cache, so they see every
  // folded key.
  if (threadIdx.x >= 64) return;
  const int i = threadIdx.x;
  const bool node = i < T;
  int p = -1, tk = 0, c = 0;
  if (node) {
    const u64 key = __hip_atomic_load(keys + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p = parent[i];
    tk = draft[i];
    c = (int)(0xFFFFFFFFu - (u32)key);
    target[i] = c;
    __hip_atomic_store(keys + i, (u64)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(row_count + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (i == 0) __hip_atomic_store(rows_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool bad = __any(node && (i == 0 ? p != -1 : (p < 0 || p >= i)));
  if (bad) {
    if (node) { path[i] = -1; emit[i] = -1; }
    if (i == 0) *n_emit = -1;
    return;
  }
  // Node i's own edge agrees when its token is the parent's choice; it is
  // valid when every edge of its root path agrees.  Pointer jumping over the
  // parent links: after ceil(log2 T) rounds every node has folded its whole
  // root path (ancestor -1 = done): `ok` = all edges agree, `depth` = edges.
  int anc = p;
  const int c_parent = __shfl(c, p < 0 ? 0 : p);  // every lane takes part in each exchange
  int ok = node && (i == 0 || tk == c_parent);
  int depth = i > 0 && node;
  for (int step = 1; step < T; step <<= 1) {
    const int a = anc < 0 ? i : anc;
    const int ok_a = __shfl(ok, a), depth_a = __shfl(depth, a), anc_a = __shfl(anc, a);
    if (anc >= 0) {
      ok = ok && ok_a;
      depth += depth_a;
      anc = anc_a;
    }
  }
  // deepest valid node, the smallest index among equally deep ones
  int best_key = (node && ok) ? (depth << 8) | (255 - i) : 0;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best_key = max(best_key, __shfl_xor(best_key, m));
  const int bn = 255 - (best_key & 255), d = best_key >> 8;
  // the path, root side first: lane k holds the node at depth k + 1
  int on_path = -1;
  for (int k = d - 1, n = bn; k >= 0; --k) {
    if (i == k) on_path = n;
    n = __shfl(p, n);
  }
  const int tok_on_path = __shfl(tk, on_path < 0 ? 0 : on_path);
  const int bonus = __shfl(c, bn);
  if (node) {
    path[i] = i < d ? on_path : -1;
    emit[i] = i < d ? tok_on_path : (i == d ? bonus : -1);
  }
  if (i == 0) *n_emit = d + 1;
}

}  // namespace

// ------------------------------------------------ the library's own workspace
// For callers that cannot allocate (code under stream capture, serving loops
// that forbid hipMalloc): one workspace per device in a static device array,
// shared by every call on that device.  Each call leaves it zero-filled, as
// it found it; calls that overlap on one device race on it.  In host code the
// array's name is not a device address: its address on the current device
// comes from hipGetSymbolAddress, once per device, and only that is used.
static __device__ __align__(256) unsigned char scratch[SVG_TREE_WORKSPACE_BYTES];

namespace {

__global__ __launch_bounds__(64) void k_zero_scratch(u32* p, int nwords) {
  for (int i = threadIdx.x; i < nwords; i += 64) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // the array's device address, per device (null until set up)

}  // namespace

hipError_t svg_tree_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // start from zeros once, with a kernel on the caller's stream (ahead of
    // its first use there; no memset node if the caller is capturing)
    hipLaunchKernelGGL(k_zero_scratch, dim3(1), dim3(64), 0, stream, static_cast<u32*>(p),
                       SVG_TREE_WORKSPACE_BYTES / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t svg_launch_tree_accept(const float* logits, int T, int V, const int32_t* parent, const int32_t* draft,
                                  int32_t* target, int32_t* path, int32_t* emit, int32_t* n_emit, void* workspace,
                                  hipStream_t stream) {
  // slices per row: about 8192 values each, and no more than two workgroups
  // per CU over the whole grid
  const int by_size = (V + 8191) / 8192;
  const int by_grid = std::max(1, 2 * svg_cu_count() / T);
  const int S = std::max(1, std::min(by_size, by_grid));
  const int L = ((V + S - 1) / S + 3) / 4 * 4;  // values per slice, a multiple of 4
  // workspace: row keys (u64) at byte 0, per-row counts (u32) at 256, the
  // count of completed rows at 384
  u64* keys = static_cast<u64*>(workspace);
  u32* row_count = reinterpret_cast<u32*>(static_cast<char*>(workspace) + 256);
  u32* rows_done = reinterpret_cast<u32*>(static_cast<char*>(workspace) + 384);
  const bool vec4 = V % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  if (vec4)
    hipLaunchKernelGGL(k_tree_accept<true>, dim3(T * S), dim3(kThreads), 0, stream, logits, T, V, S, L, parent,
                       draft, target, path, emit, n_emit, keys, row_count, rows_done);
  else
    hipLaunchKernelGGL(k_tree_accept<false>, dim3(T * S), dim3(kThreads), 0, stream, logits, T, V, S, L, parent,
                       draft, target, path, emit, n_emit, keys, row_count, rows_done);
  return hipGetLastError();
}
