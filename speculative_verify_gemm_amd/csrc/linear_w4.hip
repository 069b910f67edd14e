// W4A8 linear on gfx950: y[m][n] = x_scale[m] * sum_g s[n][g] * S_g[m][n],
// S_g[m][n] = sum_{k in g} xq[m][k] * (q[n][k] - z[n][g])  (exact int32).
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com).  Section "How Uzu optimizes bytes and tokens per
// pass": both operands are integers (int8 activations, 4-bit asymmetric
// weights with one scale per group) and the product runs on the int8 matrix
// path.  Section "Why batch-one decoding is memory-bound": a pass streams every
// weight once with about one multiply-add each, so the kernel is bound by HBM.
// Section "Producing several tokens from one model pass": matrix units pay off
// only with many rows (16 candidate tokens instead of 1).
//
// Two kernels read the same canonical layout (codes u8 [N][K/2], low nibble =
// even k; scales fp16 [N][K/g]; zeros u4 or fp16 per group):
//
//  * k_w4a8_dot  (M <= 2, and g = 32 at any M): VALU v_dot4_i32_i8.  A wave
//    covers 4 row slots x 16 lanes; lane (rs, b) owns 32 consecutive k of rows
//    rs, rs+4, rs+8, rs+12, so one 16-byte load per row gives 4 rows x 256 B
//    contiguous per instruction and the activation reorder is amortised over 4
//    rows.  Nibbles split into even-k / odd-k int8x4 words (and/shift/and);
//    the activation bytes are permuted to the same order with v_perm_b32.
//  * k_w4a8_mfma (M > 2, g = 64 or 128): v_mfma_i32_16x16x64_i8.  A = 16
//    tokens x 64 k of activations, B = 64 k x 16 weight rows; one MFMA chain
//    per quantization group, so its int32 result is the raw group partial P_g.
//    A second MFMA against an all-ones B gives A_g[m] = sum_{k in g} xq[m][k]
//    in the same register layout, and S_g = P_g - z * A_g.  Each lane loads
//    16 contiguous bytes (32 k) of its row; for g = 64 the two halves of the
//    wave hold different groups and v_permlane32_swap regroups them.
//
// A workgroup owns 16 output rows and the whole K range; its 8 waves split K
// and their fp32 partial sums are reduced through LDS in a fixed order, so the
// result is deterministic.
#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kWaves = 8;
constexpr int kRows = 16;  // output rows per workgroup

template <bool Z4>
SVG_DEV int load_zero(const void* w_zero, int n, int gi, int NG) {
  if constexpr (Z4) {
    const uint8_t b = reinterpret_cast<const uint8_t*>(w_zero)[(size_t)n * ((NG + 1) >> 1) + (gi >> 1)];
    return (gi & 1) ? (b >> 4) : (b & 0xF);
  } else {
    return (int)half_bits_to_float(reinterpret_cast<const uint16_t*>(w_zero)[(size_t)n * NG + gi]);
  }
}

// ------------------------------------------------------------------ GEMV
template <int MT, int G, bool Z4>
__global__ __launch_bounds__(kWaves * 64) void k_w4a8_dot(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale,
    const void* __restrict__ w_zero, int N, float* __restrict__ y, int32_t* __restrict__ dbg) {
  __shared__ float red[kWaves][MT][kRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rs = lane >> 4;  // row slot 0..3
  const int b = lane & 15;   // 32-k slice within a 512-k step
  const int n0 = blockIdx.x * kRows;
  const int NG = K / G;
  const size_t Kh = (size_t)K >> 1;
  const int nsteps = (K + 511) >> 9;

  float acc[4][MT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

  for (int st = wave; st < nsteps; st += kWaves) {
    const int kk = st * 512 + 32 * b;
    const bool kvalid = kk < K;
    // weights of the 4 rows: issue all loads first
    uint4 w[4];
    float sc[4];
    int zp[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + rs + 4 * r;
      const bool ok = kvalid && n < N;
      w[r] = ok ? load_nt16(wq + (size_t)n * Kh + (kk >> 1)) : make_uint4(0, 0, 0, 0);
      const int gi = kk / G;
      sc[r] = ok ? half_bits_to_float(w_scale[(size_t)n * NG + gi]) : 0.f;
      zp[r] = ok ? load_zero<Z4>(w_zero, n, gi, NG) : 0;
    }
    // activations: 32 codes per token, reordered to even/odd k
    u32 xe[MT][4], xo[MT][4];
    int asum[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
      if (kvalid && m < M) {
        const int8_t* p = xq + (size_t)m * K + kk;
        a0 = load16(p);
        a1 = load16(p + 16);
      }
      const u32 a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      int s = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        xe[m][t] = act_even(a[2 * t], a[2 * t + 1]);
        xo[m][t] = act_odd(a[2 * t], a[2 * t + 1]);
        s = dot4(a[2 * t], 0x01010101u, s);
        s = dot4(a[2 * t + 1], 0x01010101u, s);
      }
      asum[m] = s;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const u32 wd[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
      u32 we[4], wo[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        we[t] = nib_even(wd[t]);
        wo[t] = nib_odd(wd[t]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int p = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          p = dot4(we[t], xe[m][t], p);
          p = dot4(wo[t], xo[m][t], p);
        }
        int S = p - zp[r] * asum[m];  // this lane's share of S_g
        acc[r][m] = fmaf(sc[r], (float)S, acc[r][m]);
        if (dbg != nullptr) {
          // complete S_g over the G/32 lanes that hold one group
          if constexpr (G >= 64) S += lane_xor<1>(S);
          if constexpr (G >= 128) S += lane_xor<2>(S);
          const int n = n0 + rs + 4 * r;
          if (kvalid && n < N && m < M && (b % (G / 32)) == 0)
            dbg[((size_t)m * N + n) * NG + kk / G] = S;
        }
      }
    }
  }
  // reduce over the 16 k-slices of each row slot, then over waves
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m];
      v += lane_xorf<1>(v);
      v += lane_xorf<2>(v);
      v += lane_xorf<4>(v);
      v += lane_xorf<8>(v);
      if (b == 0) red[wave][m][rs + 4 * r] = v;
    }
  __syncthreads();
  if (threadIdx.x < MT * kRows) {
    const int m = threadIdx.x / kRows, nl = threadIdx.x % kRows;
    const int n = n0 + nl;
    if (m < M && n < N) {
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) v += red[w2][m][nl];
      y[(size_t)m * N + n] = x_scale[m] * v;
    }
  }
}

// ------------------------------------------------------------------ MFMA
SVG_DEV v4i mfma_i8(v4i a, v4i b, v4i c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }

// 16 activation codes at p (k order 0..15) -> MFMA operand in the order the
// unpacked weight nibbles arrive: k {0,2,4,6}, {1,3,5,7}, {8,10,12,14}, {9,...}.
SVG_DEV v4i act_operand(const int8_t* p, bool ok) {
  uint4 a = ok ? load16(p) : make_uint4(0, 0, 0, 0);
  v4i r;
  r[0] = (int)act_even(a.x, a.y);
  r[1] = (int)act_odd(a.x, a.y);
  r[2] = (int)act_even(a.z, a.w);
  r[3] = (int)act_odd(a.z, a.w);
  return r;
}
// Two packed words (16 nibbles, k order 0..15) -> MFMA operand.
SVG_DEV v4i w_operand(u32 p0, u32 p1) {
  v4i r;
  r[0] = (int)nib_even(p0);
  r[1] = (int)nib_odd(p0);
  r[2] = (int)nib_even(p1);
  r[3] = (int)nib_odd(p1);
  return r;
}

template <int MH, int G, bool Z4>
__global__ __launch_bounds__(kWaves * 64) void k_w4a8_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale,
    const void* __restrict__ w_zero, int N, float* __restrict__ y, int32_t* __restrict__ dbg) {
  static_assert(G == 64 || G == 128, "MFMA path handles groups of 64 and 128");
  __shared__ float red[kWaves][MH * 16][kRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;  // weight row (B column) of this lane
  const int b = lane >> 4;   // k-slot block 0..3
  const int n0 = blockIdx.x * kRows;
  const int n = n0 + nl;
  const bool nvalid = n < N;
  const int NG = K / G;
  const size_t Kh = (size_t)K >> 1;
  const int nsteps = (K + 127) >> 7;  // 128 k per step
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const v4i zero4 = {0, 0, 0, 0};

  float acc[MH][4];
#pragma unroll
  for (int h = 0; h < MH; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[h][r] = 0.f;

  for (int st = wave; st < nsteps; st += kWaves) {
    const int kbase = st * 128;
    const int kk = kbase + 32 * b;
    const uint4 w = (nvalid && kk < K) ? load_nt16(wq + (size_t)n * Kh + (kk >> 1))
                                       : make_uint4(0, 0, 0, 0);
    v4i B1, B2;
    int koff1, koff2;  // activation k offsets of this lane's slot block
    if constexpr (G == 64) {
      // lanes 0-31 hold group 2st, lanes 32-63 group 2st+1: regroup so MFMA 1
      // sees only group 2st and MFMA 2 only group 2st+1.
      const auto s0 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
      B1 = w_operand(s0[0], s1[0]);
      B2 = w_operand(s0[1], s1[1]);
      koff1 = kbase + ((b & 1) << 5) + ((b >> 1) << 4);  // b: 0,1,2,3 -> 0,32,16,48
      koff2 = koff1 + 64;
    } else {
      B1 = w_operand(w.x, w.y);
      B2 = w_operand(w.z, w.w);
      koff1 = kk;
      koff2 = kk + 16;
    }
    // scale and zero of this lane's row for the step's group(s)
    const int g1 = (G == 64) ? 2 * st : st;
    const int g2 = g1 + 1;
    const float s1 = (nvalid && g1 < NG) ? half_bits_to_float(w_scale[(size_t)n * NG + g1]) : 0.f;
    const int z1 = (nvalid && g1 < NG) ? load_zero<Z4>(w_zero, n, g1, NG) : 0;
    float s2 = 0.f;
    int z2 = 0;
    if constexpr (G == 64) {
      s2 = (nvalid && g2 < NG) ? half_bits_to_float(w_scale[(size_t)n * NG + g2]) : 0.f;
      z2 = (nvalid && g2 < NG) ? load_zero<Z4>(w_zero, n, g2, NG) : 0;
    }
#pragma unroll
    for (int h = 0; h < MH; ++h) {
      const int ma = h * 16 + nl;  // token of this lane's A row
      const bool mok = ma < M;
      const v4i A1 = act_operand(xq + (size_t)ma * K + koff1, mok && koff1 < K);
      const v4i A2 = act_operand(xq + (size_t)ma * K + koff2, mok && koff2 < K);
      if constexpr (G == 64) {
        const v4i P1 = mfma_i8(A1, B1, zero4);
        const v4i S1 = mfma_i8(A1, ones, zero4);
        const v4i P2 = mfma_i8(A2, B2, zero4);
        const v4i S2 = mfma_i8(A2, ones, zero4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e1 = P1[r] - z1 * S1[r];
          const int e2 = P2[r] - z2 * S2[r];
          acc[h][r] = fmaf(s1, (float)e1, acc[h][r]);
          acc[h][r] = fmaf(s2, (float)e2, acc[h][r]);
          if (dbg != nullptr) {
            const int m = h * 16 + 4 * b + r;
            if (m < M && nvalid) {
              if (g1 < NG) dbg[((size_t)m * N + n) * NG + g1] = e1;
              if (g2 < NG) dbg[((size_t)m * N + n) * NG + g2] = e2;
            }
          }
        }
      } else {
        const v4i P = mfma_i8(A2, B2, mfma_i8(A1, B1, zero4));
        const v4i S = mfma_i8(A2, ones, mfma_i8(A1, ones, zero4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = P[r] - z1 * S[r];
          acc[h][r] = fmaf(s1, (float)e, acc[h][r]);
          if (dbg != nullptr) {
            const int m = h * 16 + 4 * b + r;
            if (m < M && nvalid && g1 < NG) dbg[((size_t)m * N + n) * NG + g1] = e;
          }
        }
      }
    }
  }
  // C layout: lane holds rows m = 16h + 4b + r of column n = nl.
#pragma unroll
  for (int h = 0; h < MH; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][h * 16 + 4 * b + r][nl] = acc[h][r];
  __syncthreads();
  for (int t = threadIdx.x; t < MH * 16 * kRows; t += kWaves * 64) {
    const int m = t / kRows, c = t % kRows;
    const int nn = n0 + c;
    if (m < M && nn < N) {
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) v += red[w2][m][c];
      y[(size_t)m * N + nn] = x_scale[m] * v;
    }
  }
}

template <int MT, int G, bool Z4>
hipError_t launch_dot(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                      const uint16_t* w_scale, const void* w_zero, int N, float* y, int32_t* dbg,
                      hipStream_t stream) {
  const dim3 grid((N + kRows - 1) / kRows), block(kWaves * 64);
  hipLaunchKernelGGL((k_w4a8_dot<MT, G, Z4>), grid, block, 0, stream, xq, x_scale, M, K, wq,
                     w_scale, w_zero, N, y, dbg);
  return hipGetLastError();
}

template <int G, bool Z4>
hipError_t dispatch_g(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                      const uint16_t* w_scale, const void* w_zero, int N, float* y, int32_t* dbg,
                      hipStream_t stream) {
  if (M <= 1) return launch_dot<1, G, Z4>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
  if (M <= kGemvMaxM)
    return launch_dot<2, G, Z4>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
  if constexpr (G == 32) {
    // no MFMA form for 32-wide groups: the dot kernel, 8 tokens per launch
    const int NG = K / G;
    for (int m0 = 0; m0 < M; m0 += 8) {
      const int mc = (M - m0) < 8 ? (M - m0) : 8;
      hipError_t e = launch_dot<8, G, Z4>(xq + (size_t)m0 * K, x_scale + m0, mc, K, wq, w_scale,
                                          w_zero, N, y + (size_t)m0 * N,
                                          dbg ? dbg + (size_t)m0 * N * NG : nullptr, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else {
    const dim3 grid((N + kRows - 1) / kRows), block(kWaves * 64);
    if (M <= 16)
      hipLaunchKernelGGL((k_w4a8_mfma<1, G, Z4>), grid, block, 0, stream, xq, x_scale, M, K, wq,
                         w_scale, w_zero, N, y, dbg);
    else
      hipLaunchKernelGGL((k_w4a8_mfma<2, G, Z4>), grid, block, 0, stream, xq, x_scale, M, K, wq,
                         w_scale, w_zero, N, y, dbg);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t svg_launch_w4a8(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                           const uint16_t* w_scale, const void* w_zero, bool z4, int group, int N,
                           float* y, int32_t* dbg, hipStream_t stream) {
#define SVG_G_CASE(G)                                                                          \
  if (group == G)                                                                              \
    return z4 ? dispatch_g<G, true>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream) \
              : dispatch_g<G, false>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
  SVG_G_CASE(32)
  SVG_G_CASE(64)
  SVG_G_CASE(128)
#undef SVG_G_CASE
  return hipErrorInvalidValue;
}
