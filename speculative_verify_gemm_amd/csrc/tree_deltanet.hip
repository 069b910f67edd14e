// Rollback-free verification of a draft tree through a gated delta-rule
// layer, and the commit of the accepted path, on gfx950.
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com), section "Verifying a draft tree without restoring
// model state": a Gated DeltaNet layer keeps a fixed-size state that every
// token changes; verification computes what every branch of the draft tree
// needs without changing the live state, and only the accepted tokens'
// updates are applied afterwards.  The recurrence (not on the pages) is the
// gated delta rule of the Gated DeltaNet publication: per head, a state S of
// d_v x d_k values and, per token, S' = alpha S (I - beta k k^T) + beta v k^T
// and o = S' q.
//
// Verification: one workgroup per (node, head, row block) replays the node's root path
// from the live state, which it only reads, and writes the node's output.
// Nodes share no work, so the whole tree is one launch with no ordering
// between workgroups; the replays cost (depth + 1) d_v d_k multiply-adds
// each, which at the tree sizes of a verify pass (<= 32 nodes) is far below
// the cost of reading the state.  Commit: one workgroup per (head, row block) replays the
// root and the accepted path (as the acceptance step wrote it) and stores the
// state in place.
//
// Mapping: the rows of a state evolve independently (row r only needs itself,
// k and v[r]), so a head's d_v rows are split over d_v / 32 workgroups of 256
// threads; 8 threads share a row, each holding d_k / 8 consecutive values in
// registers for the whole replay, and a row's dot products with k and q are
// reduced across its 8 consecutive lanes.  The path's tokens are staged in LDS first (one burst of
// loads), so the replay is bound by arithmetic and LDS, not by memory latency.
#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxNodes = 32;

constexpr int kRowsPerGroup = 32;  // state rows per workgroup: rows evolve independently

template <int DK, int DV>
struct Layout {
  static constexpr int TPR = kThreads / kRowsPerGroup;  // threads per state row (8)
  static constexpr int EPT = DK / TPR;                  // values per thread
  static constexpr int GROUPS = DV / kRowsPerGroup;     // workgroups per head
  static_assert(DV % kRowsPerGroup == 0 && DK % TPR == 0 && EPT % 4 == 0, "unsupported head size");
};

template <int TPR>
SVG_DEV float row_sum(float v) {
  if constexpr (TPR >= 2) v += __shfl_xor(v, 1);
  if constexpr (TPR >= 4) v += __shfl_xor(v, 2);
  if constexpr (TPR >= 8) v += __shfl_xor(v, 4);
  return v;
}

// One token through the rule for this thread's slice: S <- alpha S +
// beta (v_r - alpha (S k)_r) k, with (S k)_r the row's full dot product.
template <int TPR, int EPT>
SVG_DEV void gdn_advance(float (&S)[EPT], const float* __restrict__ k, float v_r, float alpha, float beta,
                         int c0) {
  float kk[EPT];
#pragma unroll
  for (int c = 0; c < EPT; c += 4) {
    const float4 t = *reinterpret_cast<const float4*>(k + c0 + c);
    kk[c] = t.x; kk[c + 1] = t.y; kk[c + 2] = t.z; kk[c + 3] = t.w;
  }
  float u = 0.f;
#pragma unroll
  for (int c = 0; c < EPT; ++c) u = fmaf(S[c], kk[c], u);
  u = row_sum<TPR>(u);
  const float w = beta * (v_r - alpha * u);
#pragma unroll
  for (int c = 0; c < EPT; ++c) S[c] = fmaf(w, kk[c], alpha * S[c]);
}

// The tokens of a path (this head's k, v, alpha, beta), staged in LDS by the
// whole workgroup with all loads in flight at once: the replay then waits on
// LDS only, not on one memory round trip per token.
template <int DK, int DV>
struct Tokens {
  float k[kMaxNodes * DK];
  float v[kMaxNodes * kRowsPerGroup];  // this workgroup's rows of each value
  float a[kMaxNodes], b[kMaxNodes];
};

template <int DK, int DV>
SVG_DEV void stage_tokens(const int* nodes, int len, const float* __restrict__ k, const float* __restrict__ v,
                          const float* __restrict__ alpha, const float* __restrict__ beta, int H, int h,
                          int row0, Tokens<DK, DV>& tok) {
  for (int i = threadIdx.x; i < len * (DK / 4); i += kThreads) {
    const int j = i / (DK / 4), c = i % (DK / 4);
    reinterpret_cast<float4*>(tok.k)[i] =
        reinterpret_cast<const float4*>(k + ((size_t)nodes[j] * H + h) * DK)[c];
  }
  for (int i = threadIdx.x; i < len * kRowsPerGroup; i += kThreads) {
    const int j = i / kRowsPerGroup, c = i % kRowsPerGroup;
    tok.v[i] = v[((size_t)nodes[j] * H + h) * DV + row0 + c];
  }
  if ((int)threadIdx.x < len) {
    const size_t th = (size_t)nodes[threadIdx.x] * H + h;
    tok.a[threadIdx.x] = alpha[th];
    tok.b[threadIdx.x] = beta[th];
  }
  __syncthreads();
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_gdn_tree_verify(const float* __restrict__ state,
                                                             const float* __restrict__ q,
                                                             const float* __restrict__ k,
                                                             const float* __restrict__ v,
                                                             const float* __restrict__ alpha,
                                                             const float* __restrict__ beta,
                                                             const int32_t* __restrict__ parent, int T, int H,
                                                             float* __restrict__ out) {
  using Lo = Layout<DK, DV>;
  __shared__ int path[kMaxNodes];
  __shared__ int len;
  __shared__ Tokens<DK, DV> tok;
  const int node = blockIdx.x, h = blockIdx.y, row0 = blockIdx.z * kRowsPerGroup;
  const int rl = threadIdx.x / Lo::TPR, r = row0 + rl, c0 = (threadIdx.x % Lo::TPR) * Lo::EPT;
  // the state rows do not depend on the path: requested before its walk
  float S[Lo::EPT];
  const float* s0 = state + ((size_t)h * DV + r) * DK + c0;
#pragma unroll
  for (int c = 0; c < Lo::EPT; c += 4) {
    const float4 t = *reinterpret_cast<const float4*>(s0 + c);
    S[c] = t.x; S[c + 1] = t.y; S[c + 2] = t.z; S[c + 3] = t.w;
  }
  if (threadIdx.x == 0) {  // the root path, root first; -1 if it is not a tree path
    int n = node, d = 0, ok = 1;
    int rev[kMaxNodes];
    while (ok) {
      rev[d++] = n;
      if (n == 0) break;
      const int p = parent[n];
      ok = p >= 0 && p < n && d < kMaxNodes;
      n = p;
    }
    ok = ok && parent[0] == -1;
    for (int j = 0; j < d; ++j) path[j] = rev[d - 1 - j];
    len = ok ? d : -1;
  }
  __syncthreads();
  const size_t hd = (size_t)h * DK;
  if (len < 0) {  // malformed tree: the node's output is NaN
    if (c0 == 0) out[((size_t)node * H + h) * DV + r] = __builtin_nanf("");
    return;
  }
  stage_tokens<DK, DV>(path, len, k, v, alpha, beta, H, h, row0, tok);
  for (int j = 0; j < len; ++j)
    gdn_advance<Lo::TPR, Lo::EPT>(S, tok.k + j * DK, tok.v[j * kRowsPerGroup + rl], tok.a[j], tok.b[j], c0);
  const float* qq = q + ((size_t)node * H) * DK + hd + c0;
  float o = 0.f;
#pragma unroll
  for (int c = 0; c < Lo::EPT; c += 4) {
    const float4 t = *reinterpret_cast<const float4*>(qq + c);
    o = fmaf(S[c], t.x, o);
    o = fmaf(S[c + 1], t.y, o);
    o = fmaf(S[c + 2], t.z, o);
    o = fmaf(S[c + 3], t.w, o);
  }
  o = row_sum<Lo::TPR>(o);
  if (c0 == 0) out[((size_t)node * H + h) * DV + r] = o;
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_gdn_tree_commit(float* __restrict__ state,
                                                             const float* __restrict__ k,
                                                             const float* __restrict__ v,
                                                             const float* __restrict__ alpha,
                                                             const float* __restrict__ beta,
                                                             const int32_t* __restrict__ accepted,
                                                             const int32_t* __restrict__ n_emit, int T, int H) {
  using Lo = Layout<DK, DV>;
  __shared__ int nodes[kMaxNodes];
  __shared__ int len;
  __shared__ Tokens<DK, DV> tok;
  const int h = blockIdx.x, row0 = blockIdx.y * kRowsPerGroup;
  const int rl = threadIdx.x / Lo::TPR, r = row0 + rl, c0 = (threadIdx.x % Lo::TPR) * Lo::EPT;
  // this thread's part of the state rows, requested before the accepted path
  // is read (only this thread writes it back)
  float S[Lo::EPT];
  float* s0 = state + ((size_t)h * DV + r) * DK + c0;
#pragma unroll
  for (int c = 0; c < Lo::EPT; c += 4) {
    const float4 t = *reinterpret_cast<const float4*>(s0 + c);
    S[c] = t.x; S[c + 1] = t.y; S[c + 2] = t.z; S[c + 3] = t.w;
  }
  if (threadIdx.x == 0) {  // root, then the accepted nodes; nothing if they are not valid nodes
    const int n = n_emit[0];
    int ok = n >= 1 && n <= T;
    nodes[0] = 0;
    for (int j = 1; ok && j < n; ++j) {
      const int a = accepted[j - 1];
      ok = a >= 1 && a < T;
      nodes[j] = a;
    }
    len = ok ? n : 0;
  }
  __syncthreads();
  if (len == 0) return;
  stage_tokens<DK, DV>(nodes, len, k, v, alpha, beta, H, h, row0, tok);
  for (int j = 0; j < len; ++j)
    gdn_advance<Lo::TPR, Lo::EPT>(S, tok.k + j * DK, tok.v[j * kRowsPerGroup + rl], tok.a[j], tok.b[j], c0);
#pragma unroll
  for (int c = 0; c < Lo::EPT; c += 4) *reinterpret_cast<float4*>(s0 + c) = make_float4(S[c], S[c + 1], S[c + 2], S[c + 3]);
}

}  // namespace

bool svg_gdn_head_ok(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128 || dv == 256); }

#define SVG_GDN_SHAPES(X) X(64, 64) X(64, 128) X(64, 256) X(128, 64) X(128, 128) X(128, 256)

hipError_t svg_launch_gdn_tree_verify(const float* state, const float* q, const float* k, const float* v,
                                      const float* alpha, const float* beta, const int32_t* parent, int T, int H,
                                      int dk, int dv, float* out, hipStream_t stream) {
#define SVG_GDN_V(DK, DV)                                                                                      \
  if (dk == DK && dv == DV) {                                                                                  \
    hipLaunchKernelGGL((k_gdn_tree_verify<DK, DV>), dim3(T, H, DV / kRowsPerGroup), dim3(kThreads), 0, stream, \
                       state, q, k, v,                                                                         \
                       alpha, beta, parent, T, H, out);                                                        \
    return hipGetLastError();                                                                                  \
  }
  SVG_GDN_SHAPES(SVG_GDN_V)
#undef SVG_GDN_V
  return hipErrorInvalidValue;
}

hipError_t svg_launch_gdn_tree_commit(float* state, const float* k, const float* v, const float* alpha,
                                      const float* beta, const int32_t* path, const int32_t* n_emit, int T, int H,
                                      int dk, int dv, hipStream_t stream) {
#define SVG_GDN_C(DK, DV)                                                                                      \
  if (dk == DK && dv == DV) {                                                                                  \
    hipLaunchKernelGGL((k_gdn_tree_commit<DK, DV>), dim3(H, DV / kRowsPerGroup), dim3(kThreads), 0, stream,   \
                       state, k, v, alpha,                                                                     \
                       beta, path, n_emit, T, H);                                                              \
    return hipGetLastError();                                                                                  \
  }
  SVG_GDN_SHAPES(SVG_GDN_C)
#undef SVG_GDN_C
  return hipErrorInvalidValue;
}
