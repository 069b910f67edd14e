// Activation rotation and int8 quantization of one token row by one workgroup
// (any multiple of 64 threads up to 1024).  Used by the stand-alone
// act_rht_quant_i8 kernel and by the linear kernels that quantize their own
// input rows.
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com), section "How Uzu optimizes bytes and tokens per
// pass": random sign flips, then a +/-1 Hadamard on each block of 32 values,
// then 8-bit quantization on the fly.  Per token: amax = max |u|,
// sigma = amax / 127, q = clamp(rint(u / sigma), -127, 127), stored scale
// sigma / B (the transform's overall scale on both operands; 2^-5 for the
// pages' block B = 32, 2^-6 for the wave-wide block 64).
//
// Thread i holds float4 chunks i, i + NT, i + 2 NT, ... (NT threads), so a
// 32-block spans 8 consecutive lanes (a 64-block 16) and the butterfly is
// lane exchanges only.
//
// The code of every value is the one IEEE division u / sigma (correctly
// rounded) followed by round-half-to-even gives.  Dividing is slow, so the
// quotient is first estimated as t = u * (1 / sigma): |t - u/sigma| <= 2^-16
// for |u/sigma| <= 128, and the correctly rounded quotient is within 2^-18 of
// u/sigma.  Unless t lies within 2^-13 of a half-integer -- that is, unless
// |t - rint(t)| >= 1/2 - 2^-13 (t - rint(t) is exact) -- both round to the
// same integer as t, so rint(t) is the code; near a half-integer (about one
// value in 4000) the exact division decides.
#pragma once
#include "svg_device.h"

#pragma clang fp contract(off)

SVG_DEV int clamp_i(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// int8 codes of four values u for the scale sigma (> 0); rinv = 1 / sigma;
// `fast` is false when 1 / sigma is not a normal float (then every code
// divides).  The exact divisions sit behind one wave-uniform branch, taken
// only when some lane of the wave needs one: a per-lane branch is flattened
// by the compiler, and every value would then pay for the division.
SVG_DEV void act_codes4(const float u[4], float sigma, float rinv, bool fast, int q[4]) {
  float r[4];
  bool exact[4], any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = u[i] * rinv;
    r[i] = rintf(t);
    exact[i] = !fast || !(fabsf(t - r[i]) < 0.5f - 0x1p-13f);
    any = any || exact[i];
  }
  if (__any(any)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (exact[i]) r[i] = rintf(u[i] / sigma);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = clamp_i((int)r[i], -127, 127);
}

// Max over the workgroup with one barrier, for a `red` (>= 16 floats of LDS)
// that no earlier code of the kernel reads.
SVG_DEV float wg_max_once(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, red[w]);
  return r;
}

// Max over the workgroup (exact: max is order-free).  red: >= 16 floats of LDS.
SVG_DEV float wg_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();  // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, red[w]);
  return r;
}

// Rotated values of float4 chunk c of a row: loads (zeros past the row),
// sign flip, B-wide butterfly.
template <int B>
SVG_DEV void act_rotate4(rsrc_t xr, rsrc_t sr, u32 c, float e[4]) {
  const u32x4 v = bload16(xr, c * 16u);
  const int sg = (int)bload4(sr, c * 4u);
  e[0] = __uint_as_float(v[0]); e[1] = __uint_as_float(v[1]);
  e[2] = __uint_as_float(v[2]); e[3] = __uint_as_float(v[3]);
  apply_signs4(e[0], e[1], e[2], e[3], sg);
  fwht_lane4<B>(e[0], e[1], e[2], e[3]);
}

SVG_DEV u32 pack4(const int q[4]) {
  return (u32)(q[0] & 0xFF) | ((u32)(q[1] & 0xFF) << 8) | ((u32)(q[2] & 0xFF) << 16) |
         ((u32)(q[3] & 0xFF) << 24);
}

// Where act_quant_row puts its results: packed code words and the row scale.
// StoreGlobal: row m of a global code buffer of ldm rows in 32-k slabs
// (include/svgemm.h); AUX is the stores' cache policy (kSC1: written through
// for readers on other XCCs in the same launch).  StoreLds: a row of LDS
// words in k order.
template <int AUX>
struct StoreGlobalT {
  rsrc_t out, sc;
  u32 m, ldm;
  SVG_DEV StoreGlobalT(int8_t* xq, int m_, int ldm_, float* scale, int K)
      : out(make_rsrc(xq, (u32)ldm_ * (u32)K)), sc(make_rsrc(scale, 4u)), m((u32)m_), ldm((u32)ldm_) {}
  // word c holds k = 4c .. 4c + 3: slab c / 8, bytes 4 (c % 8) of the row's 32
  SVG_DEV void word(u32 c, u32 v) const {
    __builtin_amdgcn_raw_buffer_store_b32(v, out, ((c >> 3) * ldm + m) * 32u + 4u * (c & 7u), 0u, AUX);
  }
  SVG_DEV void scale(float v) const { __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), sc, 0u, 0u, AUX); }
};
using StoreGlobal = StoreGlobalT<0>;

struct StoreLds {
  u32* row;     // LDS, K/4 words
  float* sc;    // LDS
  SVG_DEV void word(u32 c, u32 v) const { row[c] = v; }
  SVG_DEV void scale(float v) const { *sc = v; }
};

// A row's raw inputs held in registers: chunks tid + NT * i, i < CPT (chunks
// past the row are zeros), and their sign words.  tid / NT default to the
// whole workgroup; a subset of its waves may hold the row instead.
template <int CPT>
struct RowRegs {
  float e[CPT][4];
  int sg[CPT];
};

// Request the loads of row x (K values) into r; nothing is waited for.
template <int CPT>
SVG_DEV void act_load_row(const float* x, int K, const int8_t* signs, RowRegs<CPT>& r,
                          u32 tid = threadIdx.x, u32 NT = blockDim.x) {
  const rsrc_t xr = make_rsrc(x, (u32)K * 4u);
  const rsrc_t sr = make_rsrc(signs, (u32)K);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const u32 c = tid + NT * i;
    const u32x4 v = bload16(xr, c * 16u);
    r.sg[i] = (int)bload4(sr, c * 4u);
    r.e[i][0] = __uint_as_float(v[0]); r.e[i][1] = __uint_as_float(v[1]);
    r.e[i][2] = __uint_as_float(v[2]); r.e[i][3] = __uint_as_float(v[3]);
  }
}

// Sign flip and butterfly (block B) of a row loaded by act_load_row; returns
// this thread's max |u|.
template <int CPT, int B = 32>
SVG_DEV float act_rotate_loaded(RowRegs<CPT>& r) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    apply_signs4(r.e[i][0], r.e[i][1], r.e[i][2], r.e[i][3], r.sg[i]);
    fwht_lane4<B>(r.e[i][0], r.e[i][1], r.e[i][2], r.e[i][3]);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(r.e[i][0]), fabsf(r.e[i][1])), fmaxf(fabsf(r.e[i][2]), fabsf(r.e[i][3]))));
  }
  return amax;
}

// Codes and scale of a rotated row whose max |u| over the row is amax (B:
// the transform block, whose overall scale 1/B the stored scale carries).
template <int CPT, class Store, int B = 32>
SVG_DEV void act_store_codes(const RowRegs<CPT>& r, int K, float amax, const Store& st,
                             u32 tid = threadIdx.x, u32 NT = blockDim.x) {
  const u32 nchunk = (u32)K >> 2;
  const float sigma = amax / 127.0f;
  const float rinv = 1.0f / sigma;
  const bool fast = sigma >= 0x1p-125f;
  if (tid == 0) st.scale(sigma * (1.0f / B));  // exact: a power of two
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const u32 c = tid + NT * i;
    if (c < nchunk) {
      int q[4] = {0, 0, 0, 0};
      if (amax > 0.f) act_codes4(r.e[i], sigma, rinv, fast, q);
      st.word(c, pack4(q));
    }
  }
}

// Rotate and quantize a row loaded by act_load_row (K <= 4 * NT * CPT); codes
// and the scale go to `st`.  Every thread of the workgroup must call it.
// ONCE: the kernel's only use of `red` (one barrier fewer).
template <int CPT, class Store, int B = 32, bool ONCE = false>
SVG_DEV void act_quant_loaded(RowRegs<CPT>& r, int K, const Store& st, float* red) {
  const float v = act_rotate_loaded<CPT, B>(r);
  const float amax = ONCE ? wg_max_once(v, red) : wg_max(v, red);
  act_store_codes<CPT, Store, B>(r, K, amax, st);
}

// Maxima of R values over the workgroup with one LDS round.  red: >= 16 * R.
template <int R>
SVG_DEV void wg_max_rows(float (&v)[R], float* red) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = wave_max(v[r]);
  __syncthreads();  // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int r = 0; r < R; ++r) red[wave * R + r] = v[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float m = red[r];
    for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w * R + r]);
    v[r] = m;
  }
}

// Rows 0..M-1 (M <= R) of X (K values each) rotated and quantized at once into
// LDS rows `out + r * stride` (words) and scales `scale[r]`: all loads issued
// together and one reduction for all rows, so the latency is one row's.
// Needs K <= 4 * NT * CPT; every thread of the workgroup must call it.
template <int R, int CPT, int B = 32>
SVG_DEV void act_quant_rows_lds(const float* X, int M, int K, const int8_t* signs, u32* out, int stride,
                                float* scale, float* red) {
  RowRegs<CPT> rr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) act_load_row<CPT>(X + (size_t)r * K, r < M ? K : 0, signs, rr[r]);
  float amax[R];
#pragma unroll
  for (int r = 0; r < R; ++r) amax[r] = act_rotate_loaded<CPT, B>(rr[r]);
  wg_max_rows<R>(amax, red);
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < M) act_store_codes<CPT, StoreLds, B>(rr[r], K, amax[r], StoreLds{out + r * stride, scale + r});
}

// Rotate (block B) and quantize row `x` (K values, K % B == 0); codes and the
// scale go to `st`.  Every thread of the workgroup must call it.  The row is
// held in registers when K <= 4 * NT * CPT (one read of the input); longer
// rows are read twice (the second pass recomputes the same rotated values).
template <int CPT, class Store, int B = 32, bool ONCE = false>
SVG_DEV void act_quant_row(const float* x, int K, const int8_t* signs, const Store& st, float* red) {
  const u32 NT = blockDim.x, nchunk = (u32)K >> 2;
  if (nchunk <= NT * CPT) {
    RowRegs<CPT> r;
    act_load_row<CPT>(x, K, signs, r);
    act_quant_loaded<CPT, Store, B, ONCE>(r, K, st, red);
    return;
  }
  const rsrc_t xr = make_rsrc(x, (u32)K * 4u);
  const rsrc_t sr = make_rsrc(signs, (u32)K);
  float amax = 0.f;
  for (u32 c = threadIdx.x; c < nchunk; c += NT) {
    float e[4];
    act_rotate4<B>(xr, sr, c, e);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3]))));
  }
  amax = ONCE ? wg_max_once(amax, red) : wg_max(amax, red);
  const float sigma = amax / 127.0f;
  const float rinv = 1.0f / sigma;
  const bool fast = sigma >= 0x1p-125f;
  if (threadIdx.x == 0) st.scale(sigma * (1.0f / B));
  for (u32 c = threadIdx.x; c < nchunk; c += NT) {
    float e[4];
    act_rotate4<B>(xr, sr, c, e);
    int q[4] = {0, 0, 0, 0};
    if (amax > 0.f) act_codes4(e, sigma, rinv, fast, q);
    st.word(c, pack4(q));
  }
}
