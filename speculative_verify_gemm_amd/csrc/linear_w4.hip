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
//  * MfmaW4 (M >= 2, g = 64 or 128): MFMA 1 takes the first run of every
//    lane (k 0..63 of the chunk), MFMA 2 the second (k 64..127).  For g = 64
//    each is exactly one quantization group; a second MFMA of the same
//    activations against a B holding -z in every byte accumulates
//    -z * sum_{k in g} xq[m][k] onto it, which closes S_g exactly with no
//    vector arithmetic.  For g = 128 all four MFMAs chain into one group.
//  * DotW4 (M = 1, and g = 32 at any M -- up to 2 tokens per launch, or 8
//    per launch after a separate quantization): v_dot4_i32_i8 on the same
//    tiles, lane (r, b) owning its two 16-k runs of row r.
//
// Workgroups are persistent (svg_stream.h): each walks 16-row tiles, its
// waves own fixed K ranges whose activation operands stay in registers across
// tiles, and the waves' fp32 partial sums are reduced through LDS in a fixed
// order, so the result is deterministic.  Padding (rows past N, k past K)
// holds code 0 and scale 0, and reads past the activation buffer return 0
// (buffer loads), so no lane needs a bounds test on the hot path.
#include "svg_device.h"
#include "svg_internal.h"
#include "svg_stream.h"

namespace {

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
// MFMA B operand holding -z in every byte (z in 0..15, so -z fits int8).
SVG_DEV v4i neg_zero_operand(int z) {
  const u32 w = __builtin_amdgcn_perm(0u, (u32)(-z), 0x00000000u);  // byte 0 of -z, 4 times
  return v4i{(int)w, (int)w, (int)w, (int)w};
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
  static_assert(U == 1 || U == 2 || U == 4, "a batch must lie inside one 512-k parameter block");
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

// Tile and block geometry shared by both policies.
struct W4Common {
  rsrc_t wr, sr, zr, xr;
  int lane, wave, waves, r, b, M, N, K, KT, KB, NG, ldm, m0;
  u32 lane16;
  const float* x_scale;
  float* y;
  int32_t* dbg;
  float* red;
  const int8_t* xlds = nullptr;  // LDS copy of the quantized rows (fused GEMV), row stride xlds_row
  int xlds_row = 0;

  template <int G, bool Z4>
  SVG_DEV void setup(const LinArgs& a, float* red_) {
    const int ntiles = (a.N + kTileRows - 1) / kTileRows;
    KT = (a.K + 127) >> 7;
    KB = (a.K + kMetaK - 1) / kMetaK;
    wr = make_rsrc(a.wq, (u32)ntiles * (u32)KT * 1024u);
    meta_rsrc<Z4>(sr, zr, a.w_scale, a.w_zero, ntiles, KB, kMetaK / G);
    xr = make_rsrc(a.xq, (u32)a.ldm * (u32)a.K);
    ldm = a.ldm;
    m0 = a.m0;
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    waves = blockDim.x >> 6;
    r = lane & 15;
    b = lane >> 4;
    lane16 = (u32)lane * 16u;
    M = a.M; N = a.N; K = a.K; NG = a.K / G;
    x_scale = a.x_scale; y = a.y; dbg = a.dbg;
    red = red_;
  }
  // Byte offset of chunk j of tile t for this lane; chunks past K read zeros.
  SVG_DEV u32 w_off(int t, int j, bool valid) const {
    return (valid && j < KT) ? ((u32)t * (u32)KT + (u32)j) * 1024u + lane16 : kOOB;
  }
  // Offset of this lane's 16-k run `run` (0: k 16b.., 1: k 64 + 16b..) of
  // activation row m in chunk j; rows past M and chunks past K read zeros (a
  // run past K lies past the buffer).  A wave's 16 rows of one run are 1 KiB
  // in two contiguous pieces (slab layout).
  SVG_DEV u32 x_off(int m, int j, int run) const {
    return (j < KT && m < M) ? act_slab_off(m0 + m, j * 128 + run * 64 + 16 * b, ldm) : kOOB;
  }
  // Sum the waves' partials of one output in a fixed order.
  SVG_DEV float wave_sum(const float* buf, int rows, int m, int c) const {
    float v = 0.f;
    for (int w2 = 0; w2 < waves; ++w2) v += buf[(w2 * rows + m) * kTileRows + c];
    return v;
  }
};

// ------------------------------------------------------------------ MFMA
// Policy of the MFMA kernel (svg_stream.h).  MH 16-token halves.
template <int MH, int G, bool Z4, bool DBG>
struct MfmaW4 : W4Common {
  static_assert(G == 64 || G == 128, "MFMA path handles groups of 64 and 128");
  static constexpr int kChunkK = 128, kActRegs = 8 * MH, kRedRows = MH * 16, kMaxTok = 16 * MH;
  static constexpr int kBatchRegs = 6, kFixedRegs = 48;
  // verify batches are quantized in a launch of their own (in the linear's
  // launch they were measured slower: the rows' registers leave one
  // workgroup per CU)
  static constexpr int kFusedRows = 0;
  static constexpr int GPC = 128 / G;  // groups per 128-k chunk
  using red_t = float;
  template <int NC>
  struct Acts {
    u32x4 a1[NC][MH], a2[NC][MH];
  };
  template <int U>
  struct Batch {
    u32x4 w[U];
    GroupParams<GPC, Z4, U> gp;
  };
  float acc[MH][4];

  template <int WAVES>
  SVG_DEV void init(const LinArgs& a, float* red_) {
    setup<G, Z4>(a, red_);
#pragma unroll
    for (int h = 0; h < MH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[h][i] = 0.f;
  }

  // AUX: cache policy of the loads (kSC1: rows published in this launch)
  template <int NC, bool LDS = false, int AUX = 0>
  SVG_DEV void load_acts(Acts<NC>& X, int j0) const {
    static_assert(!LDS, "the MFMA policy reads its activation rows from global memory");
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        X.a1[c][h] = bload16a<AUX>(xr, x_off(h * 16 + r, j0 + c, 0));
        X.a2[c][h] = bload16a<AUX>(xr, x_off(h * 16 + r, j0 + c, 1));
      }
  }

  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) B.w[u] = bload16_nt(wr, w_off(t, j0 + u, valid));
    B.gp.load(sr, zr, t, j0, r, KB, valid && j0 < KT);
  }

  template <int U, int XI, int NC>
  SVG_DEV void compute(const Batch<U>& B, const Acts<NC>& X, int t, int j0) {
    const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      const v4i B1 = run_operand(B.w[u][0], B.w[u][1]);
      const v4i B2 = run_operand(B.w[u][2], B.w[u][3]);
      const float s1 = B.gp.scale(u * GPC);
      const v4i Z1 = neg_zero_operand(B.gp.zero(u * GPC));
      const float s2 = (G == 64) ? B.gp.scale(u * GPC + 1) : 0.f;
      const v4i Z2 = (G == 64) ? neg_zero_operand(B.gp.zero(u * GPC + 1)) : Z1;
#pragma unroll
      for (int h = 0; h < MH; ++h) {
        const v4i A1 = as_v4i(X.a1[XI + u][h]);
        const v4i A2 = as_v4i(X.a2[XI + u][h]);
        // S_g = sum_k x (q - z): the codes' product, then the same
        // activations against -z in every byte, accumulated in place.
        if constexpr (G == 64) {
          const v4i e1 = mfma_i8(A1, Z1, mfma_i8(A1, B1, zero4));
          const v4i e2 = mfma_i8(A2, Z2, mfma_i8(A2, B2, zero4));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[h][i] = fmaf(s1, (float)e1[i], acc[h][i]);
            acc[h][i] = fmaf(s2, (float)e2[i], acc[h][i]);
            if constexpr (DBG) {
              const int m = h * 16 + 4 * b + i, n = t * kTileRows + r;
              if (m < M && n < N) {
                if (2 * j < NG) dbg[((size_t)m * N + n) * NG + 2 * j] = e1[i];
                if (2 * j + 1 < NG) dbg[((size_t)m * N + n) * NG + 2 * j + 1] = e2[i];
              }
            }
          }
        } else {
          const v4i e = mfma_i8(A2, Z1, mfma_i8(A1, Z1, mfma_i8(A2, B2, mfma_i8(A1, B1, zero4))));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[h][i] = fmaf(s1, (float)e[i], acc[h][i]);
            if constexpr (DBG) {
              const int m = h * 16 + 4 * b + i, n = t * kTileRows + r;
              if (m < M && n < N && j < NG) dbg[((size_t)m * N + n) * NG + j] = e[i];
            }
          }
        }
      }
    }
  }

  // Sum the waves' partials in a fixed order, scale, store; reset.  The two
  // LDS slots alternate between consecutive tiles, so one barrier per tile
  // suffices: a slot is rewritten only after every thread has passed the
  // barrier of the tile in between, i.e. finished reading it.
  SVG_DEV void finish(int t, int slot) {
    float* buf = red + slot * waves * kRedRows * kTileRows;
#pragma unroll
    for (int h = 0; h < MH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // C layout: tokens 16h + 4b + i of row r
        buf[(wave * kRedRows + h * 16 + 4 * b + i) * kTileRows + r] = acc[h][i];
        acc[h][i] = 0.f;
      }
    __syncthreads();
    for (int q = threadIdx.x; q < kRedRows * kTileRows; q += blockDim.x) {
      const int m = q / kTileRows, c = q % kTileRows;
      const int n = t * kTileRows + c;
      if (m < M && n < N) y[(size_t)m * N + n] = x_scale[m] * wave_sum(buf, kRedRows, m, c);
    }
  }
};

// ------------------------------------------------------------------ GEMV
// Policy of the dot-product kernel: MT tokens, v_dot4_i32_i8 on the same
// tiles, lane (r, b) owning the two 16-k runs of row r that the MFMA layout
// gives it.
template <int MT, int G, bool Z4, bool DBG>
struct DotW4 : W4Common {
  static constexpr int kChunkK = 128, kActRegs = 8 * MT, kRedRows = MT, kMaxTok = MT;
  static constexpr int kFusedRows = MT <= 2 ? MT : 0;  // rows a launch quantizes itself
  static constexpr int kBatchRegs = 6, kFixedRegs = 48;
  static constexpr int GPC = 128 / G;
  using red_t = float;
  template <int NC>
  struct Acts {
    u32x4 a1[NC][MT], a2[NC][MT];
  };
  template <int U>
  struct Batch {
    u32x4 w[U];
    GroupParams<GPC, Z4, U> gp;
  };
  int c1, c2;  // group within the chunk of the lane's two runs
  float acc[MT];

  template <int WAVES>
  SVG_DEV void init(const LinArgs& a, float* red_) {
    setup<G, Z4>(a, red_);
    c1 = (G == 32) ? (b >> 1) : 0;
    c2 = (G == 32) ? 2 + (b >> 1) : (G == 64 ? 1 : 0);
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
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
          const int8_t* row = xlds + m * xlds_row + j * 128 + 16 * b;
          X.a1[c][m] = j < KT ? *reinterpret_cast<const u32x4*>(row) : zero;
          X.a2[c][m] = j < KT ? *reinterpret_cast<const u32x4*>(row + 64) : zero;
        } else {
          X.a1[c][m] = bload16a<AUX>(xr, x_off(m, j0 + c, 0));
          X.a2[c][m] = bload16a<AUX>(xr, x_off(m, j0 + c, 1));
        }
      }
  }

  template <int U>
  SVG_DEV void load(Batch<U>& B, int t, int j0, bool valid) const {
#pragma unroll
    for (int u = 0; u < U; ++u) B.w[u] = bload16_nt(wr, w_off(t, j0 + u, valid));
    B.gp.load(sr, zr, t, j0, r, KB, valid && j0 < KT);
  }

  template <int U, int XI, int NC>
  SVG_DEV void compute(const Batch<U>& B, const Acts<NC>& X, int t, int j0) {
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
        const u32x4& a1 = X.a1[XI + u][m];
        const u32x4& a2 = X.a2[XI + u][m];
        int p1 = 0, p2 = 0, q1 = 0, q2 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          p1 = dot4(wl[k], a1[k], p1);
          p2 = dot4(wl[4 + k], a2[k], p2);
          q1 = dot4(a1[k], 0x01010101u, q1);
          q2 = dot4(a2[k], 0x01010101u, q2);
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
          const int n = t * kTileRows + r;
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

  SVG_DEV void finish(int t, int slot) {
    float* buf = red + slot * waves * kRedRows * kTileRows;
#pragma unroll
    for (int m = 0; m < MT; ++m) {  // sum the 4 run slots of each row, then the waves
      float v = acc[m];
      v += lane_xorf<16>(v);
      v += __int_as_float(lane_xor32(__float_as_int(v)));
      if (b == 0) buf[(wave * kRedRows + m) * kTileRows + r] = v;
      acc[m] = 0.f;
    }
    __syncthreads();
    if (threadIdx.x < MT * kTileRows) {
      const int m = threadIdx.x / kTileRows, c = threadIdx.x % kTileRows;
      const int n = t * kTileRows + c;
      if (m < M && n < N) y[(size_t)m * N + n] = x_scale[m] * wave_sum(buf, kRedRows, m, c);
    }
  }
};

// --------------------------------------------------------------- dispatch
template <int G, bool Z4, bool DBG>
hipError_t dispatch_g(const LinArgs& a, const ActIn* f, hipStream_t stream) {
  if (a.M <= 1) return launch_linear_auto<DotW4<1, G, Z4, DBG>>(a, f, stream);
  if constexpr (G == 32) {
    if (a.M <= 2) return launch_linear_auto<DotW4<2, G, Z4, DBG>>(a, f, stream);
    // no MFMA form for 32-wide groups: the dot kernel, 8 tokens per launch,
    // after a separate quantization of all rows when the input is fp32
    if (f) {
      hipError_t e = svg_launch_act_rht_quant(f->X, a.M, a.K, f->signs, f->block, const_cast<int8_t*>(a.xq),
                                              const_cast<float*>(a.x_scale), stream);
      if (e != hipSuccess) return e;
    }
    const int NG = a.K / G;
    for (int m0 = 0; m0 < a.M; m0 += 8) {
      LinArgs s = a;
      s.M = (a.M - m0) < 8 ? (a.M - m0) : 8;
      s.m0 = a.m0 + m0;
      s.x_scale = a.x_scale + m0;
      s.y = a.y + (size_t)m0 * a.N;
      s.dbg = DBG ? a.dbg + (size_t)m0 * a.N * NG : nullptr;
      hipError_t e = launch_linear_auto<DotW4<8, G, Z4, DBG>>(s, nullptr, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else {
    if (a.M <= 16) return launch_linear_auto<MfmaW4<1, G, Z4, DBG>>(a, f, stream);
    return launch_linear_auto<MfmaW4<2, G, Z4, DBG>>(a, f, stream);
  }
}

}  // namespace

hipError_t svg_launch_w4a8(const int8_t* xq, const float* x_scale, int M, int K, const uint8_t* wq,
                           const uint16_t* w_scale, const void* w_zero, bool z4, int group, int N,
                           float* y, int32_t* dbg, const float* X, const int8_t* signs, int block,
                           uint32_t* ws, hipStream_t stream) {
  const LinArgs a{xq, x_scale, M, K, wq, w_scale, w_zero, N, y, dbg, M, 0};
  const ActIn fa{X, signs, block, ws};
  const ActIn* f = X ? &fa : nullptr;
#define SVG_G_CASE(G)                                                                                  \
  if (group == G) {                                                                                    \
    if (dbg) return z4 ? dispatch_g<G, true, true>(a, f, stream) : dispatch_g<G, false, true>(a, f, stream); \
    return z4 ? dispatch_g<G, true, false>(a, f, stream) : dispatch_g<G, false, false>(a, f, stream);  \
  }
  SVG_G_CASE(32)
  SVG_G_CASE(64)
  SVG_G_CASE(128)
#undef SVG_G_CASE
  return hipErrorInvalidValue;
}
