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
// Weights are stored tiled (include/svgemm.h): a 16-row x 128-k tile is one
// contiguous KiB laid out in the lane order of v_mfma_i32_16x16x64_i8, so a
// wave reads each tile with one fully coalesced 16-byte load per lane and its
// consecutive tiles are consecutive KiB.  Lane l = 16*b + r receives row r's
// k-runs [16b, 16b+16) and [64+16b, 64+16b+16); nibbles are pre-interleaved so
// that (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are the codes of k..k+3
// and k+4..k+7 in natural order.  Activations therefore need no reordering.
//
//  * k_w4a8_mfma (M > 2, g = 64 or 128): MFMA 1 takes the first run of every
//    lane (k 0..63 of the chunk), MFMA 2 the second (k 64..127).  For g = 64
//    each is exactly one quantization group; a second MFMA against an
//    all-ones B gives A_g[m] = sum_{k in g} xq[m][k] in the same register
//    layout, and S_g = P_g - z * A_g closes the group.  For g = 128 both MFMAs
//    accumulate into one group.
//  * k_w4a8_dot (M <= 2, and g = 32 at any M): v_dot4_i32_i8 on the same
//    tiles, lane (r, b) owning its two 16-k runs of row r.
//
// A workgroup owns one 16-row tile and its whole K range; its waves split the
// K chunks into contiguous ranges, issue every load of a batch of chunks before
// using any, and reduce their fp32 partial sums through LDS in a fixed order,
// so the result is deterministic.  Padding (rows past N, k past K) holds code 0
// and scale 0, and activation reads past the buffer return 0 (buffer loads), so
// no lane needs a bounds test on the hot path.
#include <algorithm>

#include "svg_device.h"
#include "svg_internal.h"
#include "svg_stream.h"

namespace {

constexpr int kRows = 16;  // output rows per workgroup (one tile row block)

// Unpack a packed word (8 codes, pre-interleaved) to two int8x4 words.
SVG_DEV void unpack8(u32 w, u32& lo, u32& hi) {
  lo = w & 0x0F0F0F0Fu;
  hi = (w >> 4) & 0x0F0F0F0Fu;
}
// 8 packed bytes (16 codes of one run) -> MFMA operand (16 int8, k order).
SVG_DEV v4i run_operand(u32 w0, u32 w1) {
  u32 a, b, c, d;
  unpack8(w0, a, b);
  unpack8(w1, c, d);
  return v4i{(int)a, (int)b, (int)c, (int)d};
}
SVG_DEV v4i mfma_i8(v4i a, v4i b, v4i c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }
SVG_DEV v4i as_v4i(u32x4 a) { return v4i{(int)a[0], (int)a[1], (int)a[2], (int)a[3]}; }

// ---------------------------------------------------------- group params
// Scales and zeros of U consecutive 128-k chunks (GPC groups each) of one
// row, U in 1, 2, 4 and the first chunk a multiple of U.  The parameters of a
// (16-row tile, 512-k block, row) are contiguous (include/svgemm.h), so a
// batch is one aligned load per array; padding holds scale 0 and zero 0.
template <int GPC, bool Z4, int U>
struct GroupParams {
  static constexpr int NV = U * GPC;                  // values in the batch
  static constexpr int GPB = 4 * GPC;                 // values per (block, row)
  static constexpr int SBY = 2 * NV;                  // scale bytes
  static constexpr int ZBY = Z4 ? (NV >= 2 ? NV / 2 : 1) : 2 * NV;
  Bytes<SBY> s;
  Bytes<ZBY> z;
  int zshift;  // nibble offset of the first value (4-bit zeros, one value per batch)

  SVG_DEV void load(rsrc_t sr, rsrc_t zr, int tile, int j0, int r, int KB, bool valid) {
    // index of the batch's first value in the blocked order
    const u32 base = (((u32)tile * (u32)KB + (u32)(j0 >> 2)) * 16u + (u32)r) * GPB + (u32)(j0 & 3) * GPC;
    bload_bytes<SBY>(s, sr, valid ? base * 2u : kOOB);
    if constexpr (Z4) {
      zshift = base & 1;
      bload_bytes<ZBY>(z, zr, valid ? base >> 1 : kOOB);
    } else {
      zshift = 0;
      bload_bytes<ZBY>(z, zr, valid ? base * 2u : kOOB);
    }
  }
  SVG_DEV float scale(int i) const { return half_at(s.w, i); }
  SVG_DEV int zero(int i) const {
    if constexpr (Z4) return nibble_at(z.w, zshift + i);
    else return (int)half_at(z.w, i);
  }
};

// Resources over the blocked scales and zeros (always in range: padded).
template <bool Z4>
SVG_DEV void meta_rsrc(rsrc_t& sr, rsrc_t& zr, const uint16_t* w_scale, const void* w_zero, int ntiles,
                       int KB, int gpb) {
  const u32 nval = (u32)ntiles * 16u * (u32)KB * (u32)gpb;
  sr = make_rsrc(w_scale, nval * 2u);
  zr = make_rsrc(w_zero, Z4 ? nval / 2u : nval * 2u);
}

// ------------------------------------------------------------------ MFMA
// Policy of the MFMA kernel for the streaming driver (svg_stream.h).
template <int MH, int G, bool Z4, bool DBG, int WAVES>
struct MfmaW4 {
  static_assert(G == 64 || G == 128, "MFMA path handles groups of 64 and 128");
  static constexpr int GPC = 128 / G;              // groups per 128-k chunk
  template <int U>
  struct Batch {
    u32x4 w[U], a1[U][MH], a2[U][MH];
    GroupParams<GPC, Z4, U> gp;
  };
  rsrc_t wr, sr, zr, xr;
  int lane, wave, r, b, M, N, K, KT, KB, NG;
  const float* x_scale;
  float* y;
  int32_t* dbg;
  float (*red)[MH * 16][kRows];
  float acc[MH][4];

  // Loads of chunks j0..j0+U-1 of tile t.  Activation rows past M, and k past
  // the end of the last row, read zeros; k past K inside other rows reads the
  // next row, which meets code 0 and scale 0 (padding).
  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
    const u32 wo = valid ? ((u32)t * (u32)KT + (u32)j0) * 1024u + (u32)lane * 16u : kOOB;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      B.w[u] = bload16_nt(wr, wo + (u32)u * 1024u);
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const u32 xo = valid ? (u32)(h * 16 + r) * (u32)K + (u32)((j0 + u) * 128 + 16 * b) : kOOB;
        B.a1[u][h] = bload16(xr, xo);
        B.a2[u][h] = bload16(xr, xo + 64u);
      }
    }
    B.gp.load(sr, zr, t, j0, r, KB, valid);
  }

  template <int U>
  SVG_DEV void compute(const Batch<U>& B, int t, int j0) {
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      const v4i B1 = run_operand(B.w[u][0], B.w[u][1]);
      const v4i B2 = run_operand(B.w[u][2], B.w[u][3]);
      const float s1 = B.gp.scale(u * GPC);
      const int z1 = B.gp.zero(u * GPC);
      const float s2 = (G == 64) ? B.gp.scale(u * GPC + 1) : 0.f;
      const int z2 = (G == 64) ? B.gp.zero(u * GPC + 1) : 0;
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const v4i A1 = as_v4i(B.a1[u][h]);
        const v4i A2 = as_v4i(B.a2[u][h]);
        if constexpr (G == 64) {
          const v4i P1 = mfma_i8(A1, B1, zero4);
          const v4i C1 = mfma_i8(A1, ones, zero4);
          const v4i P2 = mfma_i8(A2, B2, zero4);
          const v4i C2 = mfma_i8(A2, ones, zero4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e1 = P1[i] - z1 * C1[i];
            const int e2 = P2[i] - z2 * C2[i];
            acc[h][i] = fmaf(s1, (float)e1, acc[h][i]);
            acc[h][i] = fmaf(s2, (float)e2, acc[h][i]);
            if constexpr (DBG) {
              const int m = h * 16 + 4 * b + i, n = t * kRows + r;
              if (m < M && n < N) {
                if (2 * j < NG) dbg[((size_t)m * N + n) * NG + 2 * j] = e1;
                if (2 * j + 1 < NG) dbg[((size_t)m * N + n) * NG + 2 * j + 1] = e2;
              }
            }
          }
        } else {
          const v4i P = mfma_i8(A2, B2, mfma_i8(A1, B1, zero4));
          const v4i C = mfma_i8(A2, ones, mfma_i8(A1, ones, zero4));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = P[i] - z1 * C[i];
            acc[h][i] = fmaf(s1, (float)e, acc[h][i]);
            if constexpr (DBG) {
              const int m = h * 16 + 4 * b + i, n = t * kRows + r;
              if (m < M && n < N && j < NG) dbg[((size_t)m * N + n) * NG + j] = e;
            }
          }
        }
      }
    }
  }

  // Sum the waves' partials in a fixed order, scale, store; reset.
  SVG_DEV void finish(int t) {
#pragma unroll
    for (int h = 0; h < MH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[wave][h * 16 + 4 * b + i][r] = acc[h][i];  // C layout: tokens 16h + 4b + i of row r
        acc[h][i] = 0.f;
      }
    __syncthreads();
    for (int q = threadIdx.x; q < MH * 16 * kRows; q += WAVES * 64) {
      const int m = q / kRows, c = q % kRows;
      const int n = t * kRows + c;
      if (m < M && n < N) {
        float v = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) v += red[w2][m][c];
        y[(size_t)m * N + n] = x_scale[m] * v;
      }
    }
    __syncthreads();
  }
};

template <int MH, int G, bool Z4, bool DBG, int WAVES, int U, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void k_w4a8_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale,
    const void* __restrict__ w_zero, int N, float* __restrict__ y, int32_t* __restrict__ dbg) {
  using P = MfmaW4<MH, G, Z4, DBG, WAVES>;
  __shared__ float red[WAVES][MH * 16][kRows];
  const int ntiles = (N + kRows - 1) / kRows;
  P p;
  p.KT = (K + 127) >> 7;
  p.wr = make_rsrc(wq, (u32)ntiles * (u32)p.KT * 1024u);
  p.KB = (K + kMetaK - 1) / kMetaK;
  meta_rsrc<Z4>(p.sr, p.zr, w_scale, w_zero, ntiles, p.KB, kMetaK / G);
  p.xr = make_rsrc(xq, (u32)M * (u32)K);
  p.lane = threadIdx.x & 63;
  p.wave = threadIdx.x >> 6;
  p.r = p.lane & 15;
  p.b = p.lane >> 4;
  p.M = M; p.N = N; p.K = K; p.NG = K / G;
  p.x_scale = x_scale; p.y = y; p.dbg = dbg;
  p.red = red;
#pragma unroll
  for (int h = 0; h < MH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) p.acc[h][i] = 0.f;
  const int per = (p.KT + WAVES - 1) / WAVES;
  const int sb = min(p.KT, p.wave * per);
  const int se = min(p.KT, sb + per);
  if constexpr (PIPE) stream_tiles_pipelined<P, U>(p, ntiles, sb, per / U);
  else stream_tiles_simple<P>(p, ntiles, sb, se);
}

// ------------------------------------------------------------------ GEMV
template <int MT, int G, bool Z4, bool DBG, int WAVES>
struct DotW4 {
  static constexpr int GPC = 128 / G;
  template <int U>
  struct Batch {
    u32x4 w[U], a1[U][MT], a2[U][MT];
    GroupParams<GPC, Z4, U> gp;
  };
  rsrc_t wr, sr, zr, xr;
  int lane, wave, r, b, M, N, K, KT, KB, NG, c1, c2;
  const float* x_scale;
  float* y;
  int32_t* dbg;
  float (*red)[MT][kRows];
  float acc[MT];

  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
    const u32 wo = valid ? ((u32)t * (u32)KT + (u32)j0) * 1024u + (u32)lane * 16u : kOOB;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      B.w[u] = bload16_nt(wr, wo + (u32)u * 1024u);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32 xo = valid ? (u32)m * (u32)K + (u32)((j0 + u) * 128 + 16 * b) : kOOB;
        B.a1[u][m] = bload16(xr, xo);
        B.a2[u][m] = bload16(xr, xo + 64u);
      }
    }
    B.gp.load(sr, zr, t, j0, r, KB, valid);
  }

  template <int U>
  SVG_DEV void compute(const Batch<U>& B, int t, int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      u32 wl[8];
      unpack8(B.w[u][0], wl[0], wl[1]);
      unpack8(B.w[u][1], wl[2], wl[3]);
      unpack8(B.w[u][2], wl[4], wl[5]);
      unpack8(B.w[u][3], wl[6], wl[7]);
      float sf1, sf2;
      int z1, z2;
      if constexpr (G == 32) {  // the lane's runs sit in groups b/2 and 2 + b/2 of the chunk
        const bool hi = c1 & 1;
        sf1 = hi ? B.gp.scale(u * 4 + 1) : B.gp.scale(u * 4);
        sf2 = hi ? B.gp.scale(u * 4 + 3) : B.gp.scale(u * 4 + 2);
        z1 = hi ? B.gp.zero(u * 4 + 1) : B.gp.zero(u * 4);
        z2 = hi ? B.gp.zero(u * 4 + 3) : B.gp.zero(u * 4 + 2);
      } else {
        sf1 = B.gp.scale(u * GPC + c1);
        sf2 = B.gp.scale(u * GPC + c2);
        z1 = B.gp.zero(u * GPC + c1);
        z2 = B.gp.zero(u * GPC + c2);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int p1 = 0, p2 = 0, q1 = 0, q2 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          p1 = dot4(wl[k], B.a1[u][m][k], p1);
          p2 = dot4(wl[4 + k], B.a2[u][m][k], p2);
          q1 = dot4(B.a1[u][m][k], 0x01010101u, q1);
          q2 = dot4(B.a2[u][m][k], 0x01010101u, q2);
        }
        int S1 = p1 - z1 * q1;  // this lane's share of its groups' S_g
        int S2 = p2 - z2 * q2;
        acc[m] = fmaf(sf1, (float)S1, acc[m]);
        acc[m] = fmaf(sf2, (float)S2, acc[m]);
        if constexpr (DBG) {
          // a group's runs: g32 -> lanes b, b^1; g64 -> all 4 b; g128 -> both runs of all 4 b
          if constexpr (G == 128) S1 += S2;
          S1 += lane_xor16(S1);
          S2 += lane_xor16(S2);
          if constexpr (G >= 64) {
            S1 += lane_xor32(S1);
            S2 += lane_xor32(S2);
          }
          const int n = t * kRows + r;
          if (m < M && n < N) {
            const int g1 = j * GPC + c1, g2 = j * GPC + c2;
            const bool lead = (G == 32) ? ((b & 1) == 0) : (b == 0);
            if (lead && g1 < NG) dbg[((size_t)m * N + n) * NG + g1] = S1;
            if (G != 128 && lead && g2 < NG) dbg[((size_t)m * N + n) * NG + g2] = S2;
          }
        }
      }
    }
  }

  SVG_DEV void finish(int t) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {  // sum the 4 run slots of each row, then the waves
      float v = acc[m];
      v += lane_xorf<16>(v);
      v += __int_as_float(lane_xor32(__float_as_int(v)));
      if (b == 0) red[wave][m][r] = v;
      acc[m] = 0.f;
    }
    __syncthreads();
    if (threadIdx.x < MT * kRows) {
      const int m = threadIdx.x / kRows, c = threadIdx.x % kRows;
      const int n = t * kRows + c;
      if (m < M && n < N) {
        float v = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) v += red[w2][m][c];
        y[(size_t)m * N + n] = x_scale[m] * v;
      }
    }
    __syncthreads();
  }
};

template <int MT, int G, bool Z4, bool DBG, int WAVES, int U, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void k_w4a8_dot(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale,
    const void* __restrict__ w_zero, int N, float* __restrict__ y, int32_t* __restrict__ dbg) {
  using P = DotW4<MT, G, Z4, DBG, WAVES>;
  __shared__ float red[WAVES][MT][kRows];
  const int ntiles = (N + kRows - 1) / kRows;
  P p;
  p.KT = (K + 127) >> 7;
  p.wr = make_rsrc(wq, (u32)ntiles * (u32)p.KT * 1024u);
  p.KB = (K + kMetaK - 1) / kMetaK;
  meta_rsrc<Z4>(p.sr, p.zr, w_scale, w_zero, ntiles, p.KB, kMetaK / G);
  p.xr = make_rsrc(xq, (u32)M * (u32)K);
  p.lane = threadIdx.x & 63;
  p.wave = threadIdx.x >> 6;
  p.r = p.lane & 15;
  p.b = p.lane >> 4;
  p.M = M; p.N = N; p.K = K; p.NG = K / G;
  p.c1 = (G == 32) ? (p.b >> 1) : 0;  // group within the chunk of the lane's two runs
  p.c2 = (G == 32) ? 2 + (p.b >> 1) : (G == 64 ? 1 : 0);
  p.x_scale = x_scale; p.y = y; p.dbg = dbg;
  p.red = red;
#pragma unroll
  for (int m = 0; m < MT; ++m) p.acc[m] = 0.f;
  const int per = (p.KT + WAVES - 1) / WAVES;
  const int sb = min(p.KT, p.wave * per);
  const int se = min(p.KT, sb + per);
  if constexpr (PIPE) stream_tiles_pipelined<P, U>(p, ntiles, sb, per / U);
  else stream_tiles_simple<P>(p, ntiles, sb, se);
}

// --------------------------------------------------------------- launching
// Persistent grid: as many workgroups as fit on the device at once (at most
// one per tile); each walks tiles with a stride of the grid size.
template <auto KERNEL>
int resident_blocks(int block) {
  static int per_cu = 0;  // one per kernel: its occupancy is fixed when it is built
  if (per_cu == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, KERNEL, block, 0) != hipSuccess || v < 1) v = 1;
    per_cu = v;
  }
  return per_cu * svg_cu_count();
}

template <auto KERNEL>
hipError_t launch_persistent(int waves, int ntiles, hipStream_t stream, const int8_t* xq,
                             const float* x_scale, int M, int K, const uint8_t* wq,
                             const uint16_t* w_scale, const void* w_zero, int N, float* y,
                             int32_t* dbg) {
  const int block = waves * 64;
  const int grid = std::max(1, std::min(ntiles, resident_blocks<KERNEL>(block)));
  auto kernel = KERNEL;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, xq, x_scale, M, K, wq, w_scale,
                     w_zero, N, y, dbg);
  return hipGetLastError();
}

// Launch shape for KT chunks per tile and `ntiles` tiles: 4 waves per tile
// and U-chunk batches when there are many tiles; 16 waves with single-chunk
// batches when tiles are few (the waves then split K finer); a plain loop
// otherwise.  Pipelined shapes need every wave to own the same even number of
// batches.
enum class Shape { kWide, kDeep, kSimple };
inline Shape pick_shape(int KT, int ntiles, int UW) {
  const bool wide_ok = KT % 4 == 0 && (KT / 4) % (2 * UW) == 0;
  const bool deep_ok = KT % 16 == 0 && (KT / 16) % 2 == 0;
  if (ntiles >= 512 && wide_ok) return Shape::kWide;
  if (deep_ok) return Shape::kDeep;
  if (wide_ok) return Shape::kWide;
  return Shape::kSimple;
}

template <int MT, int G, bool Z4, bool DBG>
hipError_t launch_dot(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                      const uint16_t* w_scale, const void* w_zero, int N, float* y, int32_t* dbg,
                      hipStream_t stream) {
  const int KT = (K + 127) >> 7, ntiles = (N + kRows - 1) / kRows;
  constexpr int UW = MT >= 8 ? 1 : 4;
  switch (pick_shape(KT, ntiles, UW)) {
    case Shape::kWide:
      return launch_persistent<k_w4a8_dot<MT, G, Z4, DBG, 4, UW, true>>(4, ntiles, stream, xq, x_scale, M,
                               K, wq, w_scale, w_zero, N, y, dbg);
    case Shape::kDeep:
      return launch_persistent<k_w4a8_dot<MT, G, Z4, DBG, 16, 1, true>>(16, ntiles, stream, xq, x_scale,
                               M, K, wq, w_scale, w_zero, N, y, dbg);
    default:
      return launch_persistent<k_w4a8_dot<MT, G, Z4, DBG, 4, 1, false>>(4, ntiles, stream, xq, x_scale, M,
                               K, wq, w_scale, w_zero, N, y, dbg);
  }
}

template <int MH, int G, bool Z4, bool DBG>
hipError_t launch_mfma(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                       const uint16_t* w_scale, const void* w_zero, int N, float* y, int32_t* dbg,
                       hipStream_t stream) {
  const int KT = (K + 127) >> 7, ntiles = (N + kRows - 1) / kRows;
  constexpr int UW = MH == 1 ? 4 : 2;
  switch (pick_shape(KT, ntiles, UW)) {
    case Shape::kWide:
      return launch_persistent<k_w4a8_mfma<MH, G, Z4, DBG, 4, UW, true>>(4, ntiles, stream, xq, x_scale,
                               M, K, wq, w_scale, w_zero, N, y, dbg);
    case Shape::kDeep:
      return launch_persistent<k_w4a8_mfma<MH, G, Z4, DBG, 16, 1, true>>(16, ntiles, stream, xq, x_scale,
                               M, K, wq, w_scale, w_zero, N, y, dbg);
    default:
      return launch_persistent<k_w4a8_mfma<MH, G, Z4, DBG, 4, 1, false>>(4, ntiles, stream, xq, x_scale,
                               M, K, wq, w_scale, w_zero, N, y, dbg);
  }
}

template <int G, bool Z4, bool DBG>
hipError_t dispatch_g(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                      const uint16_t* w_scale, const void* w_zero, int N, float* y, int32_t* dbg,
                      hipStream_t stream) {
  if (M <= 1) return launch_dot<1, G, Z4, DBG>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
  if (M <= kGemvMaxM)
    return launch_dot<2, G, Z4, DBG>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
  if constexpr (G == 32) {
    // no MFMA form for 32-wide groups: the dot kernel, 8 tokens per launch
    const int NG = K / G;
    for (int m0 = 0; m0 < M; m0 += 8) {
      const int mc = (M - m0) < 8 ? (M - m0) : 8;
      hipError_t e = launch_dot<8, G, Z4, DBG>(xq + (size_t)m0 * K, x_scale + m0, mc, K, wq, w_scale,
                                               w_zero, N, y + (size_t)m0 * N,
                                               DBG ? dbg + (size_t)m0 * N * NG : nullptr, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else {
    if (M <= 16) return launch_mfma<1, G, Z4, DBG>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
    return launch_mfma<2, G, Z4, DBG>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);
  }
}

}  // namespace

hipError_t svg_launch_w4a8(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                           const uint16_t* w_scale, const void* w_zero, bool z4, int group, int N,
                           float* y, int32_t* dbg, hipStream_t stream) {
#define SVG_G_CASE(G)                                                                                  \
  if (group == G) {                                                                                    \
    if (dbg)                                                                                           \
      return z4 ? dispatch_g<G, true, true>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream)   \
                : dispatch_g<G, false, true>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream); \
    return z4 ? dispatch_g<G, true, false>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream)    \
              : dispatch_g<G, false, false>(xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, stream);  \
  }
  SVG_G_CASE(32)
  SVG_G_CASE(64)
  SVG_G_CASE(128)
#undef SVG_G_CASE
  return hipErrorInvalidValue;
}
