// Internal launchers behind the C ABI (svgemm.h).  Each enqueues its kernels
// on `stream` and returns hipGetLastError(); argument checks are done by the
// caller in svgemm.hip before any of these is reached.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// `block`: the transform block, 32 or 64 (checked by the caller).
hipError_t svg_launch_act_rht_quant(const float* X, int M, int K, const int8_t* signs, int block, int8_t* xq,
                                    float* x_scale, hipStream_t stream);
hipError_t svg_launch_rot_quant_w4(const float* W, int N, int K, const int8_t* signs, int block, int group,
                                   bool z4, uint8_t* wq, uint16_t* w_scale, void* w_zero,
                                   float* w_rot, hipStream_t stream);
hipError_t svg_launch_rot_quant_w8(const float* W, int N, int K, const int8_t* signs, int block, int8_t* wq,
                                   uint16_t* w_scale, float* w_rot, hipStream_t stream);
// The linears read int8 codes xq / x_scale; with X != nullptr they first
// produce them from the fp32 rows X (signs, transform block), writing xq /
// x_scale as outputs (inside the linear's own launch for M = 1, in a launch
// of their own before it otherwise).
hipError_t svg_launch_w4a8(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                           const uint16_t* w_scale, const void* w_zero, bool z4, int group, int N,
                           float* y, int32_t* dbg, const float* X, const int8_t* signs, int block,
                           uint32_t* ws, hipStream_t stream);
hipError_t svg_launch_w8a8(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                           const uint16_t* w_scale, int N, float* y, int32_t* dbg, const float* X,
                           const int8_t* signs, int block, uint32_t* ws, hipStream_t stream);

// Greedy acceptance of a draft tree (tree_accept.hip); `workspace` is the
// caller's zero-filled SVG_TREE_WORKSPACE_BYTES, left zero-filled.
hipError_t svg_launch_tree_accept(const float* logits, int T, int V, const int32_t* parent, const int32_t* draft,
                                  int32_t* target, int32_t* path, int32_t* emit, int32_t* n_emit, void* workspace,
                                  hipStream_t stream);
// The device address of the library's own tree workspace on the current
// device (set up and zero-filled on `stream` at the first call per device).
hipError_t svg_tree_scratch(hipStream_t stream, void** out);

// Gated delta-rule layer over a draft tree (tree_deltanet.hip).  Head sizes:
// d_k in {64, 128}, d_v in {64, 128, 256}.
bool svg_gdn_head_ok(int dk, int dv);
hipError_t svg_launch_gdn_tree_verify(const float* state, const float* q, const float* k, const float* v,
                                      const float* alpha, const float* beta, const int32_t* parent, int T, int H,
                                      int dk, int dv, float* out, hipStream_t stream);
hipError_t svg_launch_gdn_tree_commit(float* state, const float* k, const float* v, const float* alpha,
                                      const float* beta, const int32_t* path, const int32_t* n_emit, int T, int H,
                                      int dk, int dv, hipStream_t stream);

// One pass of dependent W4A8 linears in one launch (pass.hip).  check:
// validates the steps, sizes the plan image and the workspace; returns an
// error text (and the status in *code) or nullptr.  write: the plan image into
// host memory.  launch: one persistent launch of the uploaded image.
struct svg_pass_step;
const char* svg_pass_check(const svg_pass_step* steps, int nsteps, int M, int fmt, int group, int block,
                           uint64_t* plan_bytes, uint64_t* ws_bytes, int* code);
void svg_pass_write(const svg_pass_step* steps, int nsteps, int M, int fmt, int group, int block, void* plan_host);
hipError_t svg_launch_pass(const void* plan, int M, int fmt, int group, void* ws, hipStream_t stream);

// Layout conversions (layout.hip): canonical row-major arrays <-> storage.
hipError_t svg_launch_import_weights(int fmt_w8, int z4, int group, int N, int K, const void* codes,
                                     const uint16_t* scale, const void* zero, void* wq, uint16_t* w_scale,
                                     void* w_zero, hipStream_t stream);
hipError_t svg_launch_export_weights(int fmt_w8, int z4, int group, int N, int K, const void* wq,
                                     const uint16_t* w_scale, const void* w_zero, void* codes, uint16_t* scale,
                                     void* zero, hipStream_t stream);
hipError_t svg_launch_act_codes(int to_slab, const int8_t* src, int M, int K, int8_t* dst, hipStream_t stream);

// Bytes of the weight storage (include/svgemm.h describes the layout).
// W4 codes: tiled, rows padded to 16 and K to 128.  Scales and zeros:
// blocked per (16-row tile, 512-k block, row), rows padded to 16 and K to
// 512.  W8 codes: tiled, rows padded to 16, K to 64; scales [N].
constexpr int kMetaK = 512;
inline void svg_w4_storage(int N, int K, int group, bool z4, size_t* wq_bytes, size_t* scale_bytes,
                           size_t* zero_bytes) {
  const size_t Np = (size_t)(N + 15) / 16 * 16, KT = (size_t)(K + 127) / 128;
  const size_t Gp = (size_t)(K + kMetaK - 1) / kMetaK * (kMetaK / group);  // padded groups per row
  *wq_bytes = Np * KT * 64;
  *scale_bytes = Np * Gp * 2;
  *zero_bytes = z4 ? Np * Gp / 2 : Np * Gp * 2;
}
inline void svg_w8_storage(int N, int K, size_t* wq_bytes, size_t* scale_bytes) {
  const size_t Np = (size_t)(N + 15) / 16 * 16, KT = (size_t)(K + 63) / 64;
  *wq_bytes = Np * KT * 64;
  *scale_bytes = (size_t)N * 2;
}

// Compute units of the current device (cached per device id).
int svg_cu_count();

// The dot-product (GEMV) kernels serve M = 1, and every M with 32-wide groups
// (which have no MFMA form: two tokens per launch, or eight per launch after a
// separate quantization); larger M use MFMA, whose matrix pipe is otherwise
// idle, with the rows past M zero.
