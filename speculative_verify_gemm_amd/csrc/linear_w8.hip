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
//  * DotW8  (M = 1): v_dot4_i32_i8 on the tiles.
//  * MfmaW8 (M >= 2; two 16-token halves above 16): v_mfma_i32_16x16x64_i8 chained over K; A = 16
//    tokens x 64 k, B = 64 k x 16 rows, both in natural k order.
//
// Workgroups walk the 16-row tiles persistently (svg_stream.h): waves own
// fixed K ranges whose activation operands stay in registers across tiles, and
// the int32 partials are summed through LDS (exact, so deterministic).
// Padding holds code 0; activation reads past the buffer return 0.
#include "svg_device.h"
#include "svg_internal.h"
#include "svg_stream.h"

namespace {

// Geometry shared by both policies.  W8 tiles are 16 rows x 64 k; lane
// 16b + r holds row r, k in [16b, 16b+16) of the chunk.
struct W8Common {
  rsrc_t wr, xr;
  int lane, wave, waves, r, b, M, N, K, KT, ldm, m0;
  u32 lane16;
  const float* x_scale;
  const uint16_t* w_scale;
  float* y;
  int32_t* dbg;
  int* red;
  const int8_t* xlds = nullptr;  // LDS copy of the quantized rows (fused GEMV), row stride xlds_row
  int xlds_row = 0;

  SVG_DEV void setup(const LinArgs& a, int* red_) {
    const int ntiles = (a.N + kTileRows - 1) / kTileRows;
    KT = (a.K + 63) >> 6;
    wr = make_rsrc(a.wq, (u32)ntiles * (u32)KT * 1024u);
    xr = make_rsrc(a.xq, (u32)a.ldm * (u32)a.K);
    ldm = a.ldm;
    m0 = a.m0;
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    waves = blockDim.x >> 6;
    r = lane & 15;
    b = lane >> 4;
    lane16 = (u32)lane * 16u;
    M = a.M; N = a.N; K = a.K;
    x_scale = a.x_scale; w_scale = a.w_scale; y = a.y; dbg = a.dbg;
    red = red_;
  }
  // Chunks past K read zeros.
  SVG_DEV u32 w_off(int t, int j, bool valid) const {
    return (valid && j < KT) ? ((u32)t * (u32)KT + (u32)j) * 1024u + lane16 : kOOB;
  }
  // This lane's 16 codes of activation row m in chunk j (k 64j + 16b ..);
  // rows past M and chunks past K read zeros (slab layout: a wave's 16 rows
  // are 1 KiB in two contiguous pieces).
  SVG_DEV u32 x_off(int m, int j) const {
    return (j < KT && m < M) ? act_slab_off(m0 + m, j * 64 + 16 * b, ldm) : kOOB;
  }
  // Sum the waves' partials of one output (exact), scale, store.
  SVG_DEV void store(const int* buf, int rows, int m, int c, int t) const {
    const int n = t * kTileRows + c;
    if (m < M && n < N) {
      int S = 0;
      for (int w2 = 0; w2 < waves; ++w2) S += buf[(w2 * rows + m) * kTileRows + c];
      if (dbg) dbg[(size_t)m * N + n] = S;
      y[(size_t)m * N + n] = x_scale[m] * half_bits_to_float(w_scale[n]) * (float)S;
    }
  }
};

template <int MT>
struct DotW8 : W8Common {
  static constexpr int kChunkK = 64, kActRegs = 4 * MT, kRedRows = MT, kMaxTok = MT;
  static constexpr int kFusedRows = MT <= 2 ? MT : 0;  // rows a launch quantizes itself
  static constexpr int kBatchRegs = 4, kFixedRegs = 36;
  using red_t = int;
  template <int NC>
  struct Acts {
    u32x4 a[NC][MT];
  };
  template <int U>
  struct Batch {
    u32x4 w[U];
  };
  int acc[MT];

  template <int WAVES>
  SVG_DEV void init(const LinArgs& a, int* red_) {
    setup(a, red_);
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0;
  }
  template <int NC, bool LDS = false, int AUX = 0>
  SVG_DEV void load_acts(Acts<NC>& X, int j0) const {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if constexpr (LDS) {  // rows past M and k past K are zero in the copy
          const int j = j0 + c;
          const u32x4 zero = {0u, 0u, 0u, 0u};
          X.a[c][m] = j < KT ? *reinterpret_cast<const u32x4*>(xlds + m * xlds_row + j * 64 + 16 * b) : zero;
        } else {
          X.a[c][m] = bload16a<AUX>(xr, x_off(m, j0 + c));
        }
      }
  }
  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) B.w[u] = bload16_nt(wr, w_off(t, j0 + u, valid));
  }
  template <int U, int XI, int NC>
  SVG_DEV void compute(const Batch<U>& B, const Acts<NC>& X, int, int) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4& a = X.a[XI + u][m];
        int p = acc[m];
        p = dot4(B.w[u][0], a[0], p);
        p = dot4(B.w[u][1], a[1], p);
        p = dot4(B.w[u][2], a[2], p);
        p = dot4(B.w[u][3], a[3], p);
        acc[m] = p;
      }
  }
  // One barrier per tile: the two LDS slots alternate between tiles.
  SVG_DEV void finish(int t, int slot) {
    int* buf = red + slot * waves * kRedRows * kTileRows;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      int v = acc[m];
      v += lane_xor16(v);
      v += lane_xor32(v);
      if (b == 0) buf[(wave * kRedRows + m) * kTileRows + r] = v;
      acc[m] = 0;
    }
    __syncthreads();
    if (threadIdx.x < MT * kTileRows) store(buf, kRedRows, threadIdx.x / kTileRows, threadIdx.x % kTileRows, t);
  }
};

template <int MH>
struct MfmaW8 : W8Common {
  static constexpr int kChunkK = 64, kActRegs = 4 * MH, kRedRows = MH * 16, kMaxTok = 16 * MH;
  static constexpr int kFusedRows = 0;  // verify batches are quantized in a launch of their own
  static constexpr int kBatchRegs = 4, kFixedRegs = 36;
  using red_t = int;
  template <int NC>
  struct Acts {
    u32x4 a[NC][MH];
  };
  template <int U>
  struct Batch {
    u32x4 w[U];
  };
  v4i acc[MH];

  template <int WAVES>
  SVG_DEV void init(const LinArgs& a, int* red_) {
    setup(a, red_);
#pragma unroll
    for (int h = 0; h < MH; ++h) acc[h] = v4i{0, 0, 0, 0};
  }
  template <int NC, bool LDS = false, int AUX = 0>
  SVG_DEV void load_acts(Acts<NC>& X, int j0) const {
    static_assert(!LDS, "the MFMA policy reads its activation rows from global memory");
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < MH; ++h) X.a[c][h] = bload16a<AUX>(xr, x_off(h * 16 + r, j0 + c));
  }
  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) B.w[u] = bload16_nt(wr, w_off(t, j0 + u, valid));
  }
  template <int U, int XI, int NC>
  SVG_DEV void compute(const Batch<U>& B, const Acts<NC>& X, int, int) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v4i W = {(int)B.w[u][0], (int)B.w[u][1], (int)B.w[u][2], (int)B.w[u][3]};
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const u32x4& a = X.a[XI + u][h];
        const v4i A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
        acc[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, W, acc[h], 0, 0, 0);
      }
    }
  }
  SVG_DEV void finish(int t, int slot) {
    int* buf = red + slot * waves * kRedRows * kTileRows;
#pragma unroll
    for (int h = 0; h < MH; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) buf[(wave * kRedRows + h * 16 + 4 * b + i) * kTileRows + r] = acc[h][i];
      acc[h] = v4i{0, 0, 0, 0};
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kRedRows * kTileRows; q += blockDim.x)
      store(buf, kRedRows, q / kTileRows, q % kTileRows, t);
  }
};

}  // namespace

hipError_t svg_launch_w8a8(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                           const uint16_t* w_scale, int N, float* y, int32_t* dbg, const float* X,
                           const int8_t* signs, int block, uint32_t* ws, hipStream_t stream) {
  const LinArgs a{xq, x_scale, M, K, wq, w_scale, nullptr, N, y, dbg, M, 0};
  const ActIn fa{X, signs, block, ws};
  const ActIn* f = X ? &fa : nullptr;
  if (M <= 1) return launch_linear_auto<DotW8<1>>(a, f, stream);
  if (M <= 16) return launch_linear_auto<MfmaW8<1>>(a, f, stream);
  return launch_linear_auto<MfmaW8<2>>(a, f, stream);
}
