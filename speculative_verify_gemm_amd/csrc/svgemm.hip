// C ABI entry points (include/svgemm.h): host-side validation, then one
// enqueue on the caller's stream.  No allocation, no synchronisation, no state
// shared between calls apart from the per-thread error text and the static
// workspace of tree_accept_greedy_static (one per device, tree_accept.hip).
#include "../../include/svgemm.h"

#include <stdint.h>

#include <atomic>
#include <cstdio>
#include <string>

#include "svg_internal.h"

namespace {

thread_local std::string g_last_error;

svg_status fail(svg_status code, const char* fn, const char* what) {
  g_last_error = std::string(fn) + ": " + what;
  return code;
}

svg_status ok() {
  g_last_error.clear();
  return SVG_OK;
}

svg_status hip_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return ok();
  g_last_error = std::string(fn) + ": HIP error " + std::to_string((int)e) + " (" +
                 hipGetErrorName(e) + "): " + hipGetErrorString(e);
  return SVG_EHIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }

// Transform blocks: the pages' 32, and 64 (one wave of 64 lanes, 16 of them
// per block).
bool block_ok(int b) { return b == 32 || b == 64; }

constexpr int kMaxM = 32;
constexpr int kMaxKW8 = 131072;  // 127^2 * K < 2^31
constexpr int kMaxK = 1 << 24;   // row offsets of the activation buffers stay 32-bit
constexpr int kMaxV = 1 << 30;   // vocabulary of the tree acceptance (slice arithmetic in int)

// The kernels address each weight array through one buffer resource (32-bit
// byte range): a matrix whose codes, scales or zeros reach 4 GiB is refused.
bool fits_w4(int N, int K, int group, bool z4) {
  size_t w, s, z;
  svg_w4_storage(N, K, group, z4, &w, &s, &z);
  return w < (1ull << 32) && s < (1ull << 32) && z < (1ull << 32);
}
bool fits_w8(int N, int K) {
  size_t w, s;
  svg_w8_storage(N, K, &w, &s);
  return w < (1ull << 32) && s < (1ull << 32);
}

}  // namespace

int svg_cu_count() {
  static std::atomic<int> counts[64];  // per device; every calling thread finds the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int c = counts[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 1;
    counts[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

extern "C" {

const char* svg_last_error(void) { return g_last_error.c_str(); }

svg_status svg_weight_sizes(int N, int K, int fmt, int group, uint64_t* wq_bytes,
                            uint64_t* scale_bytes, uint64_t* zero_bytes) {
  static const char* fn = "svg_weight_sizes";
  if (N < 0 || K <= 0) return fail(SVG_EINVAL, fn, "N < 0 or K <= 0");
  if (!wq_bytes || !scale_bytes || !zero_bytes) return fail(SVG_EINVAL, fn, "null output pointer");
  if (fmt != SVG_W4_ASYM_Z4 && fmt != SVG_W4_ASYM_Z16 && fmt != SVG_W8_SYM)
    return fail(SVG_EUNSUPPORTED, fn, "unknown fmt");
  if (K % 32) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32");
  size_t w, sc, z = 0;
  if (fmt == SVG_W8_SYM) {
    svg_w8_storage(N, K, &w, &sc);
  } else {
    if (!group_ok(group)) return fail(SVG_EUNSUPPORTED, fn, "group must be 32, 64 or 128");
    if (K % group) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of group");
    svg_w4_storage(N, K, group, fmt == SVG_W4_ASYM_Z4, &w, &sc, &z);
  }
  *wq_bytes = w;
  *scale_bytes = sc;
  *zero_bytes = z;
  return ok();
}

svg_status rht_rotate_weights(const float* W, int N, int K, const int8_t* signs, int block, int fmt,
                              int group, void* wq, uint16_t* w_scale, void* w_zero,
                              float* w_rot_debug, void* stream) {
  static const char* fn = "rht_rotate_weights";
  if (N < 0) return fail(SVG_EINVAL, fn, "N < 0");
  if (K <= 0) return fail(SVG_EINVAL, fn, "K <= 0");
  if (fmt != SVG_W4_ASYM_Z4 && fmt != SVG_W4_ASYM_Z16 && fmt != SVG_W8_SYM)
    return fail(SVG_EUNSUPPORTED, fn, "unknown fmt");
  if (!block_ok(block)) return fail(SVG_EUNSUPPORTED, fn, "block must be 32 or 64");
  if (K % 32) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32");
  if (K % block) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of block");
  const bool w4 = fmt != SVG_W8_SYM;
  if (w4 && !group_ok(group)) return fail(SVG_EUNSUPPORTED, fn, "group must be 32, 64 or 128");
  if (w4 && K % group) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of group");
  if (K > kMaxK) return fail(SVG_EUNSUPPORTED, fn, "K > 2^24");
  if (w4 ? !fits_w4(N, K, group, fmt == SVG_W4_ASYM_Z4) : !fits_w8(N, K))
    return fail(SVG_EUNSUPPORTED, fn, "weight storage of 4 GiB or more: split the matrix along N");
  if (!W || !signs || !wq || !w_scale || (w4 && !w_zero))
    return fail(SVG_EINVAL, fn, "null required pointer");
  if (!aligned(W, 16) || !aligned(wq, 16)) return fail(SVG_EALIGN, fn, "W and wq need 16-byte alignment");
  if (!aligned(signs, 4)) return fail(SVG_EALIGN, fn, "signs needs 4-byte alignment");
  if (!aligned(w_scale, 4) || (fmt == SVG_W4_ASYM_Z16 && !aligned(w_zero, 4)))
    return fail(SVG_EALIGN, fn, "w_scale / fp16 w_zero need 4-byte alignment");
  if (w_rot_debug && !aligned(w_rot_debug, 16)) return fail(SVG_EALIGN, fn, "w_rot_debug needs 16-byte alignment");
  if (N == 0) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (w4)
    e = svg_launch_rot_quant_w4(W, N, K, signs, block, group, fmt == SVG_W4_ASYM_Z4,
                                reinterpret_cast<uint8_t*>(wq), w_scale, w_zero, w_rot_debug, s);
  else
    e = svg_launch_rot_quant_w8(W, N, K, signs, block, reinterpret_cast<int8_t*>(wq), w_scale, w_rot_debug, s);
  return hip_status(fn, e);
}

svg_status act_rht_quant_i8(const float* X, int M, int K, const int8_t* signs, int block,
                            int8_t* xq, float* x_scale, void* stream) {
  static const char* fn = "act_rht_quant_i8";
  if (M < 0) return fail(SVG_EINVAL, fn, "M < 0");
  if (K <= 0) return fail(SVG_EINVAL, fn, "K <= 0");
  if (!block_ok(block)) return fail(SVG_EUNSUPPORTED, fn, "block must be 32 or 64");
  if (K % 32) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32");
  if (K % block) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of block");
  if (K > kMaxK) return fail(SVG_EUNSUPPORTED, fn, "K > 2^24");
  if (M > kMaxM) return fail(SVG_EUNSUPPORTED, fn, "M > 32");
  if (!X || !signs || !xq || !x_scale) return fail(SVG_EINVAL, fn, "null required pointer");
  if (!aligned(X, 16) || !aligned(xq, 16)) return fail(SVG_EALIGN, fn, "X and xq need 16-byte alignment");
  if (!aligned(signs, 4) || !aligned(x_scale, 4)) return fail(SVG_EALIGN, fn, "signs / x_scale need 4-byte alignment");
  if (M == 0) return ok();
  return hip_status(fn, svg_launch_act_rht_quant(X, M, K, signs, block, xq, x_scale,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

svg_status check_w4(const char* fn, const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                    const uint16_t* w_scale, const void* w_zero, int fmt, int group, int N, float* y,
                    int32_t* partials_debug) {
  if (M < 0 || N < 0) return fail(SVG_EINVAL, fn, "M < 0 or N < 0");
  if (K <= 0) return fail(SVG_EINVAL, fn, "K <= 0");
  if (fmt != SVG_W4_ASYM_Z4 && fmt != SVG_W4_ASYM_Z16) return fail(SVG_EUNSUPPORTED, fn, "fmt must be a W4 format");
  if (!group_ok(group)) return fail(SVG_EUNSUPPORTED, fn, "group must be 32, 64 or 128");
  if (K % 32 || K % group) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32 and of group");
  if (K > kMaxK) return fail(SVG_EUNSUPPORTED, fn, "K > 2^24");
  if (!fits_w4(N, K, group, fmt == SVG_W4_ASYM_Z4))
    return fail(SVG_EUNSUPPORTED, fn, "weight storage of 4 GiB or more: split the matrix along N");
  if (M > kMaxM) return fail(SVG_EUNSUPPORTED, fn, "M > 32");
  if (!xq || !x_scale || !wq || !w_scale || !w_zero || !y) return fail(SVG_EINVAL, fn, "null required pointer");
  if (!aligned(xq, 16) || !aligned(wq, 16)) return fail(SVG_EALIGN, fn, "xq and wq need 16-byte alignment");
  if (!aligned(x_scale, 4) || !aligned(y, 4) || !aligned(w_scale, 4) ||
      (fmt == SVG_W4_ASYM_Z16 && !aligned(w_zero, 4)) || (partials_debug && !aligned(partials_debug, 4)))
    return fail(SVG_EALIGN, fn, "misaligned scale, zero, y or partials pointer");
  return SVG_OK;
}

svg_status check_w8(const char* fn, const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                    const uint16_t* w_scale, int N, float* y, int32_t* partials_debug) {
  if (M < 0 || N < 0) return fail(SVG_EINVAL, fn, "M < 0 or N < 0");
  if (K <= 0) return fail(SVG_EINVAL, fn, "K <= 0");
  if (K % 32) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32");
  if (K > kMaxKW8) return fail(SVG_EUNSUPPORTED, fn, "K > 131072 would overflow int32 partial sums");
  if (!fits_w8(N, K)) return fail(SVG_EUNSUPPORTED, fn, "weight storage of 4 GiB or more: split the matrix along N");
  if (M > kMaxM) return fail(SVG_EUNSUPPORTED, fn, "M > 32");
  if (!xq || !x_scale || !wq || !w_scale || !y) return fail(SVG_EINVAL, fn, "null required pointer");
  if (!aligned(xq, 16) || !aligned(wq, 16)) return fail(SVG_EALIGN, fn, "xq and wq need 16-byte alignment");
  if (!aligned(x_scale, 4) || !aligned(y, 4) || !aligned(w_scale, 2) ||
      (partials_debug && !aligned(partials_debug, 4)))
    return fail(SVG_EALIGN, fn, "misaligned scale, y or partials pointer");
  return SVG_OK;
}

// The fp32 input of the fused calls: X, signs and block.
svg_status check_fused_input(const char* fn, const float* X, const int8_t* signs, int block, int K) {
  if (!X || !signs) return fail(SVG_EINVAL, fn, "null required pointer");
  if (!block_ok(block)) return fail(SVG_EUNSUPPORTED, fn, "block must be 32 or 64");
  if (K % block) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of block");
  if (!aligned(X, 16)) return fail(SVG_EALIGN, fn, "X needs 16-byte alignment");
  if (!aligned(signs, 4)) return fail(SVG_EALIGN, fn, "signs needs 4-byte alignment");
  return SVG_OK;
}

}  // namespace

extern "C" {

svg_status w4a8_linear(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                       const uint16_t* w_scale, const void* w_zero, int fmt, int group, int N,
                       float* y, int32_t* partials_debug, void* stream) {
  static const char* fn = "w4a8_linear";
  svg_status st = check_w4(fn, xq, x_scale, M, K, wq, w_scale, w_zero, fmt, group, N, y, partials_debug);
  if (st != SVG_OK) return st;
  if (M == 0 || N == 0) return ok();
  return hip_status(fn, svg_launch_w4a8(xq, x_scale, M, K, wq, w_scale, w_zero, fmt == SVG_W4_ASYM_Z4,
                                        group, N, y, partials_debug, nullptr, nullptr, 32, nullptr,
                                        reinterpret_cast<hipStream_t>(stream)));
}

svg_status w8a8_linear(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                       const uint16_t* w_scale, int N, float* y, int32_t* partials_debug,
                       void* stream) {
  static const char* fn = "w8a8_linear";
  svg_status st = check_w8(fn, xq, x_scale, M, K, wq, w_scale, N, y, partials_debug);
  if (st != SVG_OK) return st;
  if (M == 0 || N == 0) return ok();
  return hip_status(fn, svg_launch_w8a8(xq, x_scale, M, K, wq, w_scale, N, y, partials_debug, nullptr,
                                        nullptr, 32, nullptr, reinterpret_cast<hipStream_t>(stream)));
}

static svg_status fused_w4(const char* fn, const float* X, int M, int K, const int8_t* signs, int block,
                           int8_t* xq, float* x_scale, const uint8_t* wq, const uint16_t* w_scale,
                           const void* w_zero, int fmt, int group, int N, float* y, int32_t* partials_debug,
                           uint32_t* ws, void* stream) {
  svg_status st = check_w4(fn, xq, x_scale, M, K, wq, w_scale, w_zero, fmt, group, N, y, partials_debug);
  if (st == SVG_OK) st = check_fused_input(fn, X, signs, block, K);
  if (st != SVG_OK) return st;
  if (M == 0) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(fn, svg_launch_act_rht_quant(X, M, K, signs, block, xq, x_scale, s));
  return hip_status(fn, svg_launch_w4a8(xq, x_scale, M, K, wq, w_scale, w_zero, fmt == SVG_W4_ASYM_Z4,
                                        group, N, y, partials_debug, X, signs, block, ws, s));
}

static svg_status fused_w8(const char* fn, const float* X, int M, int K, const int8_t* signs, int block,
                           int8_t* xq, float* x_scale, const int8_t* wq, const uint16_t* w_scale, int N, float* y,
                           int32_t* partials_debug, uint32_t* ws, void* stream) {
  svg_status st = check_w8(fn, xq, x_scale, M, K, wq, w_scale, N, y, partials_debug);
  if (st == SVG_OK) st = check_fused_input(fn, X, signs, block, K);
  if (st != SVG_OK) return st;
  if (M == 0) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N == 0) return hip_status(fn, svg_launch_act_rht_quant(X, M, K, signs, block, xq, x_scale, s));
  return hip_status(fn, svg_launch_w8a8(xq, x_scale, M, K, wq, w_scale, N, y, partials_debug, X, signs, block, ws, s));
}

static svg_status check_linear_ws(const char* fn, const void* workspace) {
  if (!workspace) return fail(SVG_EINVAL, fn, "null workspace");
  if (!aligned(workspace, 256)) return fail(SVG_EALIGN, fn, "workspace needs 256-byte alignment");
  return SVG_OK;
}

svg_status act_quant_w4a8_linear(const float* X, int M, int K, const int8_t* signs, int block,
                                 int8_t* xq, float* x_scale, const uint8_t* wq, const uint16_t* w_scale,
                                 const void* w_zero, int fmt, int group, int N, float* y,
                                 int32_t* partials_debug, void* stream) {
  return fused_w4("act_quant_w4a8_linear", X, M, K, signs, block, xq, x_scale, wq, w_scale, w_zero, fmt, group,
                  N, y, partials_debug, nullptr, stream);
}

svg_status act_quant_w8a8_linear(const float* X, int M, int K, const int8_t* signs, int block,
                                 int8_t* xq, float* x_scale, const int8_t* wq, const uint16_t* w_scale,
                                 int N, float* y, int32_t* partials_debug, void* stream) {
  return fused_w8("act_quant_w8a8_linear", X, M, K, signs, block, xq, x_scale, wq, w_scale, N, y, partials_debug,
                  nullptr, stream);
}

svg_status act_quant_w4a8_linear_ws(const float* X, int M, int K, const int8_t* signs, int block,
                                    int8_t* xq, float* x_scale, const uint8_t* wq, const uint16_t* w_scale,
                                    const void* w_zero, int fmt, int group, int N, float* y,
                                    int32_t* partials_debug, void* workspace, void* stream) {
  static const char* fn = "act_quant_w4a8_linear_ws";
  const svg_status st = check_linear_ws(fn, workspace);
  if (st != SVG_OK) return st;
  return fused_w4(fn, X, M, K, signs, block, xq, x_scale, wq, w_scale, w_zero, fmt, group, N, y, partials_debug,
                  static_cast<uint32_t*>(workspace), stream);
}

svg_status act_quant_w8a8_linear_ws(const float* X, int M, int K, const int8_t* signs, int block,
                                    int8_t* xq, float* x_scale, const int8_t* wq, const uint16_t* w_scale,
                                    int N, float* y, int32_t* partials_debug, void* workspace, void* stream) {
  static const char* fn = "act_quant_w8a8_linear_ws";
  const svg_status st = check_linear_ws(fn, workspace);
  if (st != SVG_OK) return st;
  return fused_w8(fn, X, M, K, signs, block, xq, x_scale, wq, w_scale, N, y, partials_debug,
                  static_cast<uint32_t*>(workspace), stream);
}

svg_status tree_accept_greedy(const float* logits, int T, int V, const int32_t* parent, const int32_t* draft,
                              int32_t* target, int32_t* path, int32_t* emit, int32_t* n_emit, void* workspace,
                              void* stream) {
  static const char* fn = "tree_accept_greedy";
  if (!logits || !parent || !draft || !target || !path || !emit || !n_emit || !workspace)
    return fail(SVG_EINVAL, fn, "null pointer");
  if (T < 1 || V < 1) return fail(SVG_EINVAL, fn, "T and V must be >= 1");
  if (T > SVG_TREE_MAX_NODES) return fail(SVG_EUNSUPPORTED, fn, "T > SVG_TREE_MAX_NODES");
  if (V > kMaxV) return fail(SVG_EUNSUPPORTED, fn, "V > 2^30");
  if (!aligned(logits, 4) || !aligned(parent, 4) || !aligned(draft, 4) || !aligned(target, 4) || !aligned(path, 4) ||
      !aligned(emit, 4) || !aligned(n_emit, 4))
    return fail(SVG_EALIGN, fn, "logits, parent, draft and the outputs must be 4-byte aligned");
  if (!aligned(workspace, 8)) return fail(SVG_EALIGN, fn, "workspace must be 8-byte aligned");
  return hip_status(fn, svg_launch_tree_accept(logits, T, V, parent, draft, target, path, emit, n_emit, workspace,
                                               reinterpret_cast<hipStream_t>(stream)));
}

svg_status tree_accept_greedy_static(const float* logits, int T, int V, const int32_t* parent, const int32_t* draft,
                                     int32_t* target, int32_t* path, int32_t* emit, int32_t* n_emit, void* stream) {
  static const char* fn = "tree_accept_greedy_static";
  if (!logits || !parent || !draft || !target || !path || !emit || !n_emit)
    return fail(SVG_EINVAL, fn, "null pointer");
  if (T < 1 || V < 1) return fail(SVG_EINVAL, fn, "T and V must be >= 1");
  if (T > SVG_TREE_MAX_NODES) return fail(SVG_EUNSUPPORTED, fn, "T > SVG_TREE_MAX_NODES (the static workspace's limit)");
  if (V > kMaxV) return fail(SVG_EUNSUPPORTED, fn, "V > 2^30");
  if (!aligned(logits, 4) || !aligned(parent, 4) || !aligned(draft, 4) || !aligned(target, 4) || !aligned(path, 4) ||
      !aligned(emit, 4) || !aligned(n_emit, 4))
    return fail(SVG_EALIGN, fn, "logits, parent, draft and the outputs must be 4-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  hipError_t e = svg_tree_scratch(s, &ws);
  if (e != hipSuccess) return hip_status(fn, e);
  return hip_status(fn, svg_launch_tree_accept(logits, T, V, parent, draft, target, path, emit, n_emit, ws, s));
}

svg_status svg_pass_plan(const svg_pass_step* steps, int nsteps, int M, int fmt, int group, int block,
                         void* plan_host, uint64_t plan_host_bytes, svg_pass_info* info) {
  static const char* fn = "svg_pass_plan";
  if (!info) return fail(SVG_EINVAL, fn, "null info");
  uint64_t pb = 0, wb = 0;
  int code = SVG_OK;
  const char* err = svg_pass_check(steps, nsteps, M, fmt, group, block, &pb, &wb, &code);
  if (err) return fail(code, fn, err);
  if (plan_host) {
    if (plan_host_bytes < pb) return fail(SVG_EINVAL, fn, "plan_host is smaller than info->plan_bytes");
    if (!aligned(plan_host, 8)) return fail(SVG_EALIGN, fn, "plan_host needs 8-byte alignment");
    svg_pass_write(steps, nsteps, M, fmt, group, block, plan_host);
  }
  info->nsteps = nsteps;
  info->M = M;
  info->fmt = fmt;
  info->group = group;
  info->block = block;
  info->plan_bytes = pb;
  info->workspace_bytes = wb;
  return ok();
}

svg_status svg_pass_run(const void* plan, const svg_pass_info* info, void* workspace, void* stream) {
  static const char* fn = "svg_pass_run";
  if (!plan || !info || !workspace) return fail(SVG_EINVAL, fn, "null pointer");
  if (info->nsteps < 1 || info->M < 1) return fail(SVG_EINVAL, fn, "info has nsteps < 1 or M < 1");
  if (info->M > 16 || (info->fmt != SVG_W4_ASYM_Z4 && info->fmt != SVG_W4_ASYM_Z16) ||
      (info->group != 64 && info->group != 128) || (info->block != 32 && info->block != 64))
    return fail(SVG_EUNSUPPORTED, fn, "info names an unsupported M, fmt, group or block");
  if (!aligned(plan, 8)) return fail(SVG_EALIGN, fn, "plan needs 8-byte alignment");
  if (!aligned(workspace, 256)) return fail(SVG_EALIGN, fn, "workspace needs 256-byte alignment");
  if (svg_cu_count() < 8) return fail(SVG_EUNSUPPORTED, fn, "the device has fewer than 8 compute units");
  return hip_status(fn, svg_launch_pass(plan, info->M, info->fmt, info->group, workspace,
                                        reinterpret_cast<hipStream_t>(stream)));
}

svg_status tree_deltanet_verify(const float* state, const float* q, const float* k, const float* v,
                                const float* alpha, const float* beta, const int32_t* parent, int T, int H,
                                int dk, int dv, float* out, void* stream) {
  static const char* fn = "tree_deltanet_verify";
  if (!state || !q || !k || !v || !alpha || !beta || !parent || !out) return fail(SVG_EINVAL, fn, "null pointer");
  if (T < 1 || H < 1) return fail(SVG_EINVAL, fn, "T and H must be >= 1");
  if (T > SVG_TREE_MAX_NODES || H > 65535) return fail(SVG_EUNSUPPORTED, fn, "T > SVG_TREE_MAX_NODES or H > 65535");
  if (!svg_gdn_head_ok(dk, dv)) return fail(SVG_EUNSUPPORTED, fn, "unsupported head size (dk, dv)");
  if (!aligned(state, 16) || !aligned(q, 16) || !aligned(k, 16))
    return fail(SVG_EALIGN, fn, "state, q and k need 16-byte alignment");
  if (!aligned(v, 4) || !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(parent, 4) || !aligned(out, 4))
    return fail(SVG_EALIGN, fn, "v, alpha, beta, parent and out need 4-byte alignment");
  return hip_status(fn, svg_launch_gdn_tree_verify(state, q, k, v, alpha, beta, parent, T, H, dk, dv, out,
                                                   reinterpret_cast<hipStream_t>(stream)));
}

svg_status tree_deltanet_commit(float* state, const float* k, const float* v, const float* alpha, const float* beta,
                                const int32_t* path, const int32_t* n_emit, int T, int H, int dk, int dv,
                                void* stream) {
  static const char* fn = "tree_deltanet_commit";
  if (!state || !k || !v || !alpha || !beta || !path || !n_emit) return fail(SVG_EINVAL, fn, "null pointer");
  if (T < 1 || H < 1) return fail(SVG_EINVAL, fn, "T and H must be >= 1");
  if (T > SVG_TREE_MAX_NODES || H > 65535) return fail(SVG_EUNSUPPORTED, fn, "T > SVG_TREE_MAX_NODES or H > 65535");
  if (!svg_gdn_head_ok(dk, dv)) return fail(SVG_EUNSUPPORTED, fn, "unsupported head size (dk, dv)");
  if (!aligned(state, 16) || !aligned(k, 16)) return fail(SVG_EALIGN, fn, "state and k need 16-byte alignment");
  if (!aligned(v, 4) || !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(path, 4) || !aligned(n_emit, 4))
    return fail(SVG_EALIGN, fn, "v, alpha, beta, path and n_emit need 4-byte alignment");
  return hip_status(fn, svg_launch_gdn_tree_commit(state, k, v, alpha, beta, path, n_emit, T, H, dk, dv,
                                                   reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ------------------------------------------------------ layout conversions
namespace {
// The checks both weight conversions share; `codes`, `scale` and `zero` are
// the canonical arrays, the others the storage.
svg_status weight_layout_check(const char* fn, int fmt, int group, int N, int K, const void* codes,
                               const uint16_t* scale, const void* zero, const void* wq, const uint16_t* w_scale,
                               const void* w_zero) {
  if (N < 0) return fail(SVG_EINVAL, fn, "N < 0");
  if (K <= 0) return fail(SVG_EINVAL, fn, "K <= 0");
  if (fmt != SVG_W4_ASYM_Z4 && fmt != SVG_W4_ASYM_Z16 && fmt != SVG_W8_SYM)
    return fail(SVG_EUNSUPPORTED, fn, "unknown fmt");
  if (K % 32) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32");
  const bool w4 = fmt != SVG_W8_SYM;
  if (w4 && !group_ok(group)) return fail(SVG_EUNSUPPORTED, fn, "group must be 32, 64 or 128");
  if (w4 && K % group) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of group");
  if (K > kMaxK) return fail(SVG_EUNSUPPORTED, fn, "K > 2^24");
  if (w4 ? !fits_w4(N, K, group, fmt == SVG_W4_ASYM_Z4) : !fits_w8(N, K))
    return fail(SVG_EUNSUPPORTED, fn, "weight storage of 4 GiB or more: split the matrix along N");
  if ((uint64_t)N * (uint64_t)K >= (1ull << 40)) return fail(SVG_EUNSUPPORTED, fn, "N * K too large");
  if (!codes || !scale || !wq || !w_scale || (w4 && (!zero || !w_zero)))
    return fail(SVG_EINVAL, fn, "null required pointer");
  if (!aligned(wq, 16)) return fail(SVG_EALIGN, fn, "wq needs 16-byte alignment");
  if (!aligned(w_scale, 4) || (fmt == SVG_W4_ASYM_Z16 && !aligned(w_zero, 4)))
    return fail(SVG_EALIGN, fn, "w_scale / fp16 w_zero need 4-byte alignment");
  if (!aligned(scale, 2) || (fmt == SVG_W4_ASYM_Z16 && !aligned(zero, 2)))
    return fail(SVG_EALIGN, fn, "the fp16 scale / zero rows need 2-byte alignment");
  return SVG_OK;
}
}  // namespace

extern "C" {

svg_status svg_import_weights(int fmt, int group, int N, int K, const void* codes, const uint16_t* scale,
                              const void* zero, void* wq, uint16_t* w_scale, void* w_zero, void* stream) {
  static const char* fn = "svg_import_weights";
  const svg_status st = weight_layout_check(fn, fmt, group, N, K, codes, scale, zero, wq, w_scale, w_zero);
  if (st != SVG_OK) return st;
  if (N == 0) return ok();
  return hip_status(fn, svg_launch_import_weights(fmt == SVG_W8_SYM, fmt == SVG_W4_ASYM_Z4, group, N, K, codes,
                                                  scale, zero, wq, w_scale, w_zero,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

svg_status svg_export_weights(int fmt, int group, int N, int K, const void* wq, const uint16_t* w_scale,
                              const void* w_zero, void* codes, uint16_t* scale, void* zero, void* stream) {
  static const char* fn = "svg_export_weights";
  const svg_status st = weight_layout_check(fn, fmt, group, N, K, codes, scale, zero, wq, w_scale, w_zero);
  if (st != SVG_OK) return st;
  if (N == 0) return ok();
  return hip_status(fn, svg_launch_export_weights(fmt == SVG_W8_SYM, fmt == SVG_W4_ASYM_Z4, group, N, K, wq,
                                                  w_scale, w_zero, codes, scale, zero,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

static svg_status act_layout(const char* fn, int to_slab, const int8_t* src, int M, int K, int8_t* dst,
                             void* stream) {
  if (M < 0) return fail(SVG_EINVAL, fn, "M < 0");
  if (K <= 0) return fail(SVG_EINVAL, fn, "K <= 0");
  if (K % 32) return fail(SVG_EUNSUPPORTED, fn, "K must be a multiple of 32");
  if ((uint64_t)M * (uint64_t)K >= (1ull << 34)) return fail(SVG_EUNSUPPORTED, fn, "M * K too large");
  if (!src || !dst) return fail(SVG_EINVAL, fn, "null required pointer");
  const int8_t* slab = to_slab ? dst : src;
  const int8_t* rows = to_slab ? src : dst;
  if (!aligned(slab, 16)) return fail(SVG_EALIGN, fn, "the slab codes need 16-byte alignment");
  if (!aligned(rows, 4)) return fail(SVG_EALIGN, fn, "the code rows need 4-byte alignment");
  if (M == 0) return ok();
  return hip_status(fn, svg_launch_act_codes(to_slab, src, M, K, dst, reinterpret_cast<hipStream_t>(stream)));
}

svg_status svg_import_act_codes(const int8_t* rows, int M, int K, int8_t* xq, void* stream) {
  return act_layout("svg_import_act_codes", 1, rows, M, K, xq, stream);
}

svg_status svg_export_act_codes(const int8_t* xq, int M, int K, int8_t* rows, void* stream) {
  return act_layout("svg_export_act_codes", 0, xq, M, K, rows, stream);
}

}  // extern "C"
