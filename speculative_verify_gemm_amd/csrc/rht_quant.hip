// Block-diagonal random Hadamard transform fused with quantization, gfx950.
// Every kernel takes the transform block B as a template argument: 32 (the
// pages' block) or 64 (the wave-wide variant, one more butterfly stage).
//
//  * k_act_rht_quant   -- activations: sign flip + 32-wide butterfly, per-row
//                         |u| max, int8 codes and the per-row scale (one
//                         workgroup per token row, svg_act.h).
//  * k_rot_quant_w4    -- weights, 4-bit asymmetric per group along K.
//  * k_rot_quant_w8    -- weights, 8-bit symmetric per row.
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com), section "How Uzu optimizes bytes and tokens per
// pass": random sign flips come before the mixing, each block of 32 values is
// mixed on its own by a +/-1 Hadamard, the transform precedes quantization,
// activations are quantized to 8 bits on the fly, Medium weights are 4-bit
// asymmetric and Large weights 8-bit symmetric.
//
// Mapping: a workgroup owns one row.  Each thread holds float4 chunks (4
// consecutive values), so a 32-block spans 8 consecutive lanes and the
// butterfly needs only lane exchanges (DPP and ds_swizzle), no LDS traffic.
// The weight kernels take row-wide maxima in two passes over the row (the
// second pass recomputes the transform from the L2-resident input, which is
// bit-identical), so any K is handled without holding the row in registers.
//
// Everything that decides an integer code is one IEEE fp32 operation with
// round-to-nearest-even (this file is compiled with -ffp-contract=off and
// correctly rounded division): the codes match a plain fp32 implementation of
// the same steps bit for bit.
#include "svg_act.h"
#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kThreads = 256;

// Load 4 values and their 4 signs, flip and transform (block B).  `valid` is
// uniform over each B/4-lane block because K is a multiple of B.
template <int B>
SVG_DEV void rotate_chunk(const float* __restrict__ row, const int8_t* __restrict__ signs, int c,
                          bool valid, float& e0, float& e1, float& e2, float& e3) {
  if (valid) {
    const float4 v = *reinterpret_cast<const float4*>(row + 4 * c);
    const int sg = *reinterpret_cast<const int*>(signs + 4 * c);
    e0 = v.x; e1 = v.y; e2 = v.z; e3 = v.w;
    apply_signs4(e0, e1, e2, e3, sg);
  } else {
    e0 = e1 = e2 = e3 = 0.f;
  }
  fwht_lane4<B>(e0, e1, e2, e3);
}

// Max over the workgroup (exact: max is order-free).
SVG_DEV float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

#pragma clang fp contract(off)

template <int NT, int CPT, int B>
__global__ __launch_bounds__(NT) void k_act_rht_quant(const float* __restrict__ X, int K,
                                                     const int8_t* __restrict__ signs,
                                                     int8_t* __restrict__ xq, float* __restrict__ x_scale) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  // one row per workgroup: `red` serves one maximum only
  act_quant_row<CPT, StoreGlobal, B, true>(X + (size_t)m * K, K, signs,
                                           StoreGlobal(xq, m, gridDim.x, x_scale + m, K), red);
}

// Group-wise min/max over the LPG = G/4 lanes that hold one quantization group.
template <int LPG>
SVG_DEV float group_min(float v) {
  v = fminf(v, lane_xorf<1>(v));
  v = fminf(v, lane_xorf<2>(v));
  v = fminf(v, lane_xorf<4>(v));
  if constexpr (LPG >= 16) v = fminf(v, lane_xorf<8>(v));
  if constexpr (LPG >= 32) v = fminf(v, lane_xorf<16>(v));
  return v;
}
template <int LPG>
SVG_DEV float group_max(float v) {
  v = fmaxf(v, lane_xorf<1>(v));
  v = fmaxf(v, lane_xorf<2>(v));
  v = fmaxf(v, lane_xorf<4>(v));
  if constexpr (LPG >= 16) v = fmaxf(v, lane_xorf<8>(v));
  if constexpr (LPG >= 32) v = fmaxf(v, lane_xorf<16>(v));
  return v;
}

// Byte offset of the 4-byte word holding codes k0..k0+7 (k0 % 8 == 0) of row
// n in the tiled W4 layout (see include/svgemm.h): tiles of 16 rows x 128 k,
// 1 KiB each; piece 16*b + r of a tile holds row r's k-runs [16b, 16b+16) and
// [64+16b, 64+16b+16) of the chunk.
SVG_DEV size_t w4_word_offset(int n, int k0, int KT) {
  const int i = n >> 4, r = n & 15;
  const int j = k0 >> 7, kc = k0 & 127;
  const int h = kc >> 6, b = (kc & 63) >> 4, w = (kc & 15) >> 3;
  return ((size_t)i * KT + j) * 1024 + (size_t)(16 * b + r) * 16 + h * 8 + w * 4;
}

// Index of the (row n, group g) parameter in the blocked order: the
// 512/group parameters of (16-row tile, 512-k block, row) are contiguous.
SVG_DEV size_t w4_param_index(int n, int g, int KB, int gpb) {
  const int i = n >> 4, r = n & 15, jb = g / gpb, c = g % gpb;
  return (((size_t)i * KB + jb) * 16 + r) * gpb + c;
}

template <int G, bool Z4, int B>
__global__ __launch_bounds__(kThreads) void k_rot_quant_w4(const float* __restrict__ W, int K,
                                                          const int8_t* __restrict__ signs,
                                                          uint8_t* __restrict__ wq,
                                                          uint16_t* __restrict__ w_scale,
                                                          void* __restrict__ w_zero,
                                                          float* __restrict__ w_rot) {
  constexpr int LPG = G / 4;            // lanes per group (8, 16 or 32)
  constexpr int GPB = kMetaK / G;       // groups per 512-k parameter block
  const int n = blockIdx.x;
  const int KB = (K + kMetaK - 1) / kMetaK;
  const float* row = W + (size_t)n * K;
  const int nchunk = K >> 2;
  const int KT = (K + 127) >> 7;
  const int lane = threadIdx.x & 63;
  for (int c0 = 0; c0 < nchunk; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const bool valid = c < nchunk;  // uniform over each group since K % G == 0
    float e0, e1, e2, e3;
    rotate_chunk<B>(row, signs, c, valid, e0, e1, e2, e3);
    if (w_rot != nullptr && valid)
      *reinterpret_cast<float4*>(w_rot + (size_t)n * K + 4 * c) = make_float4(e0, e1, e2, e3);
    const float mn = group_min<LPG>(fminf(fminf(e0, e1), fminf(e2, e3)));
    const float mx = group_max<LPG>(fmaxf(fmaxf(e0, e1), fmaxf(e2, e3)));
    const float lo = fminf(0.f, mn);
    const float hi = fmaxf(0.f, mx);
    __half sh = __float2half_rn((hi - lo) / 15.0f);
    if (__half_as_ushort(sh) == 0) sh = __ushort_as_half(0x3C00);  // 1.0
    const float s = __half2float(sh);
    // the zero point is a 4-bit unsigned value: -lo / s passes 15 when s
    // falls in fp16's subnormal range, whose steps are coarse
    const int z = valid ? clamp_i((int)rintf(-lo / s), 0, 15) : 0;
    const int q0 = clamp_i((int)rintf(e0 / s) + z, 0, 15);
    const int q1 = clamp_i((int)rintf(e1 / s) + z, 0, 15);
    const int q2 = clamp_i((int)rintf(e2 / s) + z, 0, 15);
    const int q3 = clamp_i((int)rintf(e3 / s) + z, 0, 15);
    // codes k = 4c..4c+3 go to the low (c even) or high (c odd) nibbles of
    // bytes 0..3 of the word covering k0 = 8*(c/2): pair adjacent lanes.
    const u32 spread = (u32)q0 | ((u32)q1 << 8) | ((u32)q2 << 16) | ((u32)q3 << 24);
    const u32 other = (u32)lane_xor<1>((int)spread);
    const int gi = c / LPG;
    const bool leader = (lane % LPG) == 0;
    int z_next = 0;
    if constexpr (Z4) z_next = lane_xor<LPG>(z);  // zero of the odd partner group
    if (valid) {
      if ((c & 1) == 0)
        *reinterpret_cast<u32*>(wq + w4_word_offset(n, 4 * c, KT)) = spread | (other << 4);
      if (leader) {
        const size_t pi = w4_param_index(n, gi, KB, GPB);
        w_scale[pi] = __half_as_ushort(sh);
        if constexpr (Z4) {
          // pairs (2c, 2c+1) of a block share a byte; the next group of a
          // block is the next group of the row (blocks hold whole pairs)
          if ((gi & 1) == 0) {
            const int zo = (gi + 1 < K / G) ? z_next : 0;
            reinterpret_cast<uint8_t*>(w_zero)[pi >> 1] = (uint8_t)(z | (zo << 4));
          }
        } else {
          reinterpret_cast<uint16_t*>(w_zero)[pi] = __half_as_ushort(__int2half_rn(z));
        }
      }
    }
  }
}

// Byte offset of codes k..k+3 (k % 4 == 0) of row n in the tiled W8 layout:
// tiles of 16 rows x 64 k; piece 16*b + r holds row r's k in [16b, 16b+16).
SVG_DEV size_t w8_offset(int n, int k, int KT8) {
  const int i = n >> 4, r = n & 15, j = k >> 6, kc = k & 63;
  return ((size_t)i * KT8 + j) * 1024 + (size_t)(16 * (kc >> 4) + r) * 16 + (kc & 15);
}

template <int B>
__global__ __launch_bounds__(kThreads) void k_rot_quant_w8(const float* __restrict__ W, int K,
                                                          const int8_t* __restrict__ signs,
                                                          int8_t* __restrict__ wq,
                                                          uint16_t* __restrict__ w_scale,
                                                          float* __restrict__ w_rot) {
  __shared__ float red[kThreads / 64];
  const int n = blockIdx.x;
  const float* row = W + (size_t)n * K;
  const int nchunk = K >> 2;
  const int KT8 = (K + 63) >> 6;
  float amax = 0.f;
  for (int c0 = 0; c0 < nchunk; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const bool valid = c < nchunk;
    float e0, e1, e2, e3;
    rotate_chunk<B>(row, signs, c, valid, e0, e1, e2, e3);
    if (valid) {
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(e0), fabsf(e1)), fmaxf(fabsf(e2), fabsf(e3))));
      if (w_rot != nullptr)
        *reinterpret_cast<float4*>(w_rot + (size_t)n * K + 4 * c) = make_float4(e0, e1, e2, e3);
    }
  }
  amax = block_max(amax, red);
  __half sh = __float2half_rn(amax / 127.0f);
  if (__half_as_ushort(sh) == 0) sh = __ushort_as_half(0x3C00);
  const float s = __half2float(sh);
  if (threadIdx.x == 0) w_scale[n] = __half_as_ushort(sh);
  for (int c0 = 0; c0 < nchunk; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const bool valid = c < nchunk;
    float e0, e1, e2, e3;
    rotate_chunk<B>(row, signs, c, valid, e0, e1, e2, e3);
    if (valid) {
      const int q0 = clamp_i((int)rintf(e0 / s), -127, 127);
      const int q1 = clamp_i((int)rintf(e1 / s), -127, 127);
      const int q2 = clamp_i((int)rintf(e2 / s), -127, 127);
      const int q3 = clamp_i((int)rintf(e3 / s), -127, 127);
      *reinterpret_cast<u32*>(wq + w8_offset(n, 4 * c, KT8)) =
          (u32)(q0 & 0xFF) | ((u32)(q1 & 0xFF) << 8) | ((u32)(q2 & 0xFF) << 16) | ((u32)(q3 & 0xFF) << 24);
    }
  }
}

// Zero-fill of a 4-byte-aligned byte range (the padding of the tiled layouts);
// a kernel rather than a memset so that a captured graph replays it safely.
__global__ __launch_bounds__(kThreads) void k_fill_zero(u32* __restrict__ p, size_t nwords) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nwords; i += (size_t)gridDim.x * kThreads)
    p[i] = 0u;
}

}  // namespace

template <int B>
static void launch_act(const float* X, int M, int K, const int8_t* signs, int8_t* xq, float* x_scale,
                       hipStream_t stream) {
  const int nchunk = K / 4;  // float4 chunks of a row
  const dim3 grid(M);
#define SVG_ACT(NT, CPT) \
  hipLaunchKernelGGL((k_act_rht_quant<NT, CPT, B>), grid, dim3(NT), 0, stream, X, K, signs, xq, x_scale)
  if (nchunk <= 256) SVG_ACT(256, 1);
  else if (nchunk <= 512) SVG_ACT(512, 1);
  else if (nchunk <= 1024) SVG_ACT(1024, 1);
  else if (nchunk <= 2048) SVG_ACT(1024, 2);
  else if (nchunk <= 3072) SVG_ACT(1024, 3);
  else if (nchunk <= 4096) SVG_ACT(1024, 4);
  else if (nchunk <= 6144) SVG_ACT(1024, 6);
  else SVG_ACT(1024, 8);  // past 8192 chunks the row is read twice
#undef SVG_ACT
}

hipError_t svg_launch_act_rht_quant(const float* X, int M, int K, const int8_t* signs, int block, int8_t* xq,
                                    float* x_scale, hipStream_t stream) {
  if (block == 64) launch_act<64>(X, M, K, signs, xq, x_scale, stream);
  else launch_act<32>(X, M, K, signs, xq, x_scale, stream);
  return hipGetLastError();
}

static hipError_t fill_zero(void* p, size_t nbytes, hipStream_t stream) {
  const size_t nwords = nbytes / 4;
  const unsigned blocks = (unsigned)((nwords + kThreads - 1) / kThreads < 1024 ? (nwords + kThreads - 1) / kThreads : 1024);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(kThreads), 0, stream, reinterpret_cast<u32*>(p), nwords);
  return hipGetLastError();
}

hipError_t svg_launch_rot_quant_w4(const float* W, int N, int K, const int8_t* signs, int block, int group,
                                   bool z4, uint8_t* wq, uint16_t* w_scale, void* w_zero,
                                   float* w_rot, hipStream_t stream) {
  if (N % 16 || K % kMetaK) {  // the tiled/blocked storage has padding: clear it first
    size_t wb, sb, zb;
    svg_w4_storage(N, K, group, z4, &wb, &sb, &zb);
    hipError_t e;
    if ((e = fill_zero(wq, wb, stream)) != hipSuccess) return e;
    if ((e = fill_zero(w_scale, sb, stream)) != hipSuccess) return e;
    if ((e = fill_zero(w_zero, zb, stream)) != hipSuccess) return e;
  }
  const dim3 grid(N), threads(kThreads);
#define SVG_W4_CASE(G, B)                                                                         \
  if (group == G && block == B) {                                                                 \
    if (z4)                                                                                       \
      hipLaunchKernelGGL((k_rot_quant_w4<G, true, B>), grid, threads, 0, stream, W, K, signs, wq, \
                         w_scale, w_zero, w_rot);                                                 \
    else                                                                                          \
      hipLaunchKernelGGL((k_rot_quant_w4<G, false, B>), grid, threads, 0, stream, W, K, signs,    \
                         wq, w_scale, w_zero, w_rot);                                             \
    return hipGetLastError();                                                                     \
  }
  SVG_W4_CASE(32, 32)
  SVG_W4_CASE(64, 32)
  SVG_W4_CASE(128, 32)
  SVG_W4_CASE(32, 64)
  SVG_W4_CASE(64, 64)
  SVG_W4_CASE(128, 64)
#undef SVG_W4_CASE
  return hipErrorInvalidValue;
}

hipError_t svg_launch_rot_quant_w8(const float* W, int N, int K, const int8_t* signs, int block, int8_t* wq,
                                   uint16_t* w_scale, float* w_rot, hipStream_t stream) {
  if (N % 16 || K % 64) {
    size_t wb, sb;
    svg_w8_storage(N, K, &wb, &sb);
    hipError_t e = fill_zero(wq, wb, stream);
    if (e != hipSuccess) return e;
  }
  if (block == 64)
    hipLaunchKernelGGL(k_rot_quant_w8<64>, dim3(N), dim3(kThreads), 0, stream, W, K, signs, wq, w_scale, w_rot);
  else
    hipLaunchKernelGGL(k_rot_quant_w8<32>, dim3(N), dim3(kThreads), 0, stream, W, K, signs, wq, w_scale, w_rot);
  return hipGetLastError();
}
