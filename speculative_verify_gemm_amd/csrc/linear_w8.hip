// W8A8 linear on gfx950: y[m][n] = x_scale[m] * s[n] * S[m][n],
// S[m][n] = sum_k xq[m][k] * q[n][k]  (exact int32; |S| <= 127^2 K < 2^31).
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com), section "How Uzu optimizes bytes and tokens per
// pass": Large checkpoints are 8-bit symmetric and both operands of the
// matmul are integers; section "Producing several tokens from one model pass":
// verification gives the matrix units 16 to 32 rows of work.
//
// Weights are int8 and tiled (include/svgemm.h): a 16-row x 64-k tile is one
// contiguous KiB in the lane order of v_mfma_i32_16x16x64_i8 (lane 16*b + r
// holds row r, k in [16b, 16b+16)), used as stored with no unpacking.  The
// integer sum closes once per row, so both kernels accumulate int32 across the
// whole K range and apply the two scales once at the end:
//
//  * k_w8a8_dot  (M <= 2): v_dot4_i32_i8 on the tiles.
//  * k_w8a8_mfma (M > 2): v_mfma_i32_16x16x64_i8 chained over K; A = 16
//    tokens x 64 k, B = 64 k x 16 rows, both in natural k order.
//
// Workgroups walk the 16-row tiles persistently (svg_stream.h); a tile's waves
// split its K chunks into contiguous ranges and the int32 partials are summed
// through LDS (exact, so deterministic).  Padding holds code 0; activation
// reads past the buffer return 0.
#include <algorithm>

#include "svg_device.h"
#include "svg_internal.h"
#include "svg_stream.h"

namespace {

constexpr int kRows = 16;

// Policies for the streaming driver (svg_stream.h).  W8 tiles are 16 rows x 64
// k; lane 16b + r holds row r, k in [16b, 16b+16) of the chunk.
template <int MT, bool DBG, int WAVES>
struct DotW8 {
  template <int U>
  struct Batch {
    u32x4 w[U], a[U][MT];
  };
  rsrc_t wr, xr;
  int lane, wave, r, b, M, N, K, KT;
  const float* x_scale;
  const uint16_t* w_scale;
  float* y;
  int32_t* dbg;
  int (*red)[MT][kRows];
  int acc[MT];

  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
    const u32 wo = valid ? ((u32)t * (u32)KT + (u32)j0) * 1024u + (u32)lane * 16u : kOOB;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      B.w[u] = bload16_nt(wr, wo + (u32)u * 1024u);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        B.a[u][m] = bload16(xr, valid ? (u32)m * (u32)K + (u32)((j0 + u) * 64 + 16 * b) : kOOB);
    }
  }
  template <int U>
  SVG_DEV void compute(const Batch<U>& B, int, int) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int p = acc[m];
        p = dot4(B.w[u][0], B.a[u][m][0], p);
        p = dot4(B.w[u][1], B.a[u][m][1], p);
        p = dot4(B.w[u][2], B.a[u][m][2], p);
        p = dot4(B.w[u][3], B.a[u][m][3], p);
        acc[m] = p;
      }
  }
  SVG_DEV void finish(int t) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      int v = acc[m];
      v += lane_xor16(v);
      v += lane_xor32(v);
      if (b == 0) red[wave][m][r] = v;
      acc[m] = 0;
    }
    __syncthreads();
    if (threadIdx.x < MT * kRows) {
      const int m = threadIdx.x / kRows, c = threadIdx.x % kRows;
      const int n = t * kRows + c;
      if (m < M && n < N) {
        int S = 0;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) S += red[w2][m][c];
        if constexpr (DBG) dbg[(size_t)m * N + n] = S;
        y[(size_t)m * N + n] = x_scale[m] * half_bits_to_float(w_scale[n]) * (float)S;
      }
    }
    __syncthreads();
  }
};

template <int MH, bool DBG, int WAVES>
struct MfmaW8 {
  template <int U>
  struct Batch {
    u32x4 w[U], a[U][MH];
  };
  rsrc_t wr, xr;
  int lane, wave, r, b, M, N, K, KT;
  const float* x_scale;
  const uint16_t* w_scale;
  float* y;
  int32_t* dbg;
  int (*red)[MH * 16][kRows];
  v4i acc[MH];

  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
    const u32 wo = valid ? ((u32)t * (u32)KT + (u32)j0) * 1024u + (u32)lane * 16u : kOOB;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      B.w[u] = bload16_nt(wr, wo + (u32)u * 1024u);
#pragma unroll
      for (int h = 0; h < MH; ++h)
        B.a[u][h] = bload16(xr, valid ? (u32)(h * 16 + r) * (u32)K + (u32)((j0 + u) * 64 + 16 * b) : kOOB);
    }
  }
  template <int U>
  SVG_DEV void compute(const Batch<U>& B, int, int) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v4i W = {(int)B.w[u][0], (int)B.w[u][1], (int)B.w[u][2], (int)B.w[u][3]};
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const v4i A = {(int)B.a[u][h][0], (int)B.a[u][h][1], (int)B.a[u][h][2], (int)B.a[u][h][3]};
        acc[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, W, acc[h], 0, 0, 0);
      }
    }
  }
  SVG_DEV void finish(int t) {
#pragma unroll
    for (int h = 0; h < MH; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][h * 16 + 4 * b + i][r] = acc[h][i];
      acc[h] = v4i{0, 0, 0, 0};
    }
    __syncthreads();
    for (int q = threadIdx.x; q < MH * 16 * kRows; q += WAVES * 64) {
      const int m = q / kRows, c = q % kRows;
      const int n = t * kRows + c;
      if (m < M && n < N) {
        int S = 0;
#pragma unroll
        for (int w2 = 0; w2 < WAVES; ++w2) S += red[w2][m][c];
        if constexpr (DBG) dbg[(size_t)m * N + n] = S;
        y[(size_t)m * N + n] = x_scale[m] * half_bits_to_float(w_scale[n]) * (float)S;
      }
    }
    __syncthreads();
  }
};

template <class P>
SVG_DEV void w8_setup(P& p, const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                      const uint16_t* w_scale, int N, float* y, int32_t* dbg, int ntiles) {
  p.KT = (K + 63) >> 6;
  p.wr = make_rsrc(wq, (u32)ntiles * (u32)p.KT * 1024u);
  p.xr = make_rsrc(xq, (u32)M * (u32)K);
  p.lane = threadIdx.x & 63;
  p.wave = threadIdx.x >> 6;
  p.r = p.lane & 15;
  p.b = p.lane >> 4;
  p.M = M; p.N = N; p.K = K;
  p.x_scale = x_scale; p.w_scale = w_scale; p.y = y; p.dbg = dbg;
}

template <int MT, bool DBG, int WAVES, int U, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void k_w8a8_dot(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const int8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale, int N,
    float* __restrict__ y, int32_t* __restrict__ dbg) {
  using P = DotW8<MT, DBG, WAVES>;
  __shared__ int red[WAVES][MT][kRows];
  const int ntiles = (N + kRows - 1) / kRows;
  P p;
  w8_setup(p, xq, x_scale, M, K, wq, w_scale, N, y, dbg, ntiles);
  p.red = red;
#pragma unroll
  for (int m = 0; m < MT; ++m) p.acc[m] = 0;
  const int per = (p.KT + WAVES - 1) / WAVES;
  const int sb = min(p.KT, p.wave * per);
  const int se = min(p.KT, sb + per);
  if constexpr (PIPE) stream_tiles_pipelined<P, U>(p, ntiles, sb, per / U);
  else stream_tiles_simple<P>(p, ntiles, sb, se);
}

template <int MH, bool DBG, int WAVES, int U, bool PIPE>
__global__ __launch_bounds__(WAVES * 64) void k_w8a8_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const int8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale, int N,
    float* __restrict__ y, int32_t* __restrict__ dbg) {
  using P = MfmaW8<MH, DBG, WAVES>;
  __shared__ int red[WAVES][MH * 16][kRows];
  const int ntiles = (N + kRows - 1) / kRows;
  P p;
  w8_setup(p, xq, x_scale, M, K, wq, w_scale, N, y, dbg, ntiles);
  p.red = red;
#pragma unroll
  for (int h = 0; h < MH; ++h) p.acc[h] = v4i{0, 0, 0, 0};
  const int per = (p.KT + WAVES - 1) / WAVES;
  const int sb = min(p.KT, p.wave * per);
  const int se = min(p.KT, sb + per);
  if constexpr (PIPE) stream_tiles_pipelined<P, U>(p, ntiles, sb, per / U);
  else stream_tiles_simple<P>(p, ntiles, sb, se);
}

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
hipError_t launch_w8(int waves, int ntiles, hipStream_t stream, const int8_t* xq, const float* x_scale,
                     int M, int K, const int8_t* wq, const uint16_t* w_scale, int N, float* y,
                     int32_t* dbg) {
  const int block = waves * 64;
  const int grid = std::max(1, std::min(ntiles, resident_blocks<KERNEL>(block)));
  auto kernel = KERNEL;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, xq, x_scale, M, K, wq, w_scale, N, y, dbg);
  return hipGetLastError();
}

// 64-k chunks: 4 waves x 8-chunk batches with many tiles, 16 waves x 2-chunk
// batches with few, a plain loop otherwise.

template <int T, bool DBG, bool MF>
hipError_t launch_w8_kind(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                          const uint16_t* w_scale, int N, float* y, int32_t* dbg, hipStream_t stream) {
  const int KT = (K + 63) >> 6, ntiles = (N + kRows - 1) / kRows;
#define SVG_W8_GO(W, U, PIPE)                                                                          \
  return MF ? launch_w8<k_w8a8_mfma<T, DBG, W, U, PIPE>>(W, ntiles, stream, xq, x_scale, M, K, wq,      \
                                                          w_scale, N, y, dbg)                          \
            : launch_w8<k_w8a8_dot<T, DBG, W, U, PIPE>>(W, ntiles, stream, xq, x_scale, M, K, wq,       \
                                                         w_scale, N, y, dbg)
  if (ntiles >= 512 && KT % 4 == 0 && (KT / 4) % 16 == 0) SVG_W8_GO(4, 8, true);
  if (KT % 16 == 0 && (KT / 16) % 4 == 0) SVG_W8_GO(16, 2, true);
  if (KT % 4 == 0 && (KT / 4) % 16 == 0) SVG_W8_GO(4, 8, true);
  SVG_W8_GO(4, 1, false);
#undef SVG_W8_GO
}

}  // namespace

hipError_t svg_launch_w8a8(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                           const uint16_t* w_scale, int N, float* y, int32_t* dbg,
                           hipStream_t stream) {
#define SVG_W8(T, MF) \
  return dbg ? launch_w8_kind<T, true, MF>(xq, x_scale, M, K, wq, w_scale, N, y, dbg, stream) \
             : launch_w8_kind<T, false, MF>(xq, x_scale, M, K, wq, w_scale, N, y, dbg, stream)
  if (M <= 1) SVG_W8(1, false);
  if (M <= kGemvMaxM) SVG_W8(2, false);
  if (M <= 16) SVG_W8(1, true);
  SVG_W8(2, true);
#undef SVG_W8
}
