// W8A8 linear on gfx950: y[m][n] = x_scale[m] * s[n] * S[m][n],
// S[m][n] = sum_k xq[m][k] * q[n][k]  (exact int32; |S| <= 127^2 K < 2^31).
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com), section "How Uzu optimizes bytes and tokens per
// pass": Large checkpoints are 8-bit symmetric and both operands of the
// matmul are integers; section "Producing several tokens from one model pass":
// verification gives the matrix units 16 to 32 rows of work.
//
// Weights are int8 [N][K] row-major, used as stored (no unpacking).  The
// integer sum closes once per row, so both kernels accumulate int32 across the
// whole K range and apply the two scales once at the end:
//
//  * k_w8a8_dot  (M <= 2): v_dot4_i32_i8; lane (rs, b) owns 16 consecutive k
//    of rows rs, rs+4, rs+8, rs+12 (4 rows x 256 B contiguous per load).
//  * k_w8a8_mfma (M > 2): v_mfma_i32_16x16x64_i8 chained over K; A = 16
//    tokens x 64 k, B = 64 k x 16 rows, both in natural k order.
//
// A workgroup owns 16 rows and all of K; its 8 waves split K and the int32
// partials are summed through LDS (exact, so the result is deterministic).
#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kWaves = 8;
constexpr int kRows = 16;

template <int MT>
__global__ __launch_bounds__(kWaves * 64) void k_w8a8_dot(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const int8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale, int N,
    float* __restrict__ y, int32_t* __restrict__ dbg) {
  __shared__ int red[kWaves][MT][kRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rs = lane >> 4;
  const int b = lane & 15;
  const int n0 = blockIdx.x * kRows;
  const int nsteps = (K + 255) >> 8;  // 256 k per step
  int acc[4][MT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0;

  for (int st = wave; st < nsteps; st += kWaves) {
    const int kk = st * 256 + 16 * b;
    const bool kvalid = kk < K;
    uint4 w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + rs + 4 * r;
      w[r] = (kvalid && n < N) ? load_nt16(wq + (size_t)n * K + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint4 a = (kvalid && m < M) ? load16(xq + (size_t)m * K + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int p = acc[r][m];
        p = dot4(w[r].x, a.x, p);
        p = dot4(w[r].y, a.y, p);
        p = dot4(w[r].z, a.z, p);
        p = dot4(w[r].w, a.w, p);
        acc[r][m] = p;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      int v = acc[r][m];
      v += lane_xor<1>(v);
      v += lane_xor<2>(v);
      v += lane_xor<4>(v);
      v += lane_xor<8>(v);
      if (b == 0) red[wave][m][rs + 4 * r] = v;
    }
  __syncthreads();
  if (threadIdx.x < MT * kRows) {
    const int m = threadIdx.x / kRows, nl = threadIdx.x % kRows;
    const int n = n0 + nl;
    if (m < M && n < N) {
      int S = 0;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) S += red[w2][m][nl];
      if (dbg != nullptr) dbg[(size_t)m * N + n] = S;
      y[(size_t)m * N + n] = x_scale[m] * half_bits_to_float(w_scale[n]) * (float)S;
    }
  }
}

template <int MH>
__global__ __launch_bounds__(kWaves * 64) void k_w8a8_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int K,
    const int8_t* __restrict__ wq, const uint16_t* __restrict__ w_scale, int N,
    float* __restrict__ y, int32_t* __restrict__ dbg) {
  __shared__ int red[kWaves][MH * 16][kRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int b = lane >> 4;
  const int n0 = blockIdx.x * kRows;
  const int n = n0 + nl;
  const bool nvalid = n < N;
  const int nsteps = (K + 63) >> 6;  // 64 k per step
  v4i acc[MH];
#pragma unroll
  for (int h = 0; h < MH; ++h) acc[h] = v4i{0, 0, 0, 0};

  for (int st = wave; st < nsteps; st += kWaves) {
    const int kk = st * 64 + 16 * b;
    const bool kvalid = kk < K;
    const uint4 w = (kvalid && nvalid) ? load_nt16(wq + (size_t)n * K + kk) : make_uint4(0, 0, 0, 0);
    const v4i B = {(int)w.x, (int)w.y, (int)w.z, (int)w.w};
#pragma unroll
    for (int h = 0; h < MH; ++h) {
      const int ma = h * 16 + nl;
      const uint4 a = (kvalid && ma < M) ? load16(xq + (size_t)ma * K + kk) : make_uint4(0, 0, 0, 0);
      const v4i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
      acc[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc[h], 0, 0, 0);
    }
  }
#pragma unroll
  for (int h = 0; h < MH; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][h * 16 + 4 * b + r][nl] = acc[h][r];
  __syncthreads();
  for (int t = threadIdx.x; t < MH * 16 * kRows; t += kWaves * 64) {
    const int m = t / kRows, c = t % kRows;
    const int nn = n0 + c;
    if (m < M && nn < N) {
      int S = 0;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) S += red[w2][m][c];
      if (dbg != nullptr) dbg[(size_t)m * N + nn] = S;
      y[(size_t)m * N + nn] = x_scale[m] * half_bits_to_float(w_scale[nn]) * (float)S;
    }
  }
}

}  // namespace

hipError_t svg_launch_w8a8(const int8_t* xq, const float* x_scale, int M, int K, const int8_t* wq,
                           const uint16_t* w_scale, int N, float* y, int32_t* dbg,
                           hipStream_t stream) {
  const dim3 grid((N + kRows - 1) / kRows), block(kWaves * 64);
  if (M <= 1)
    hipLaunchKernelGGL((k_w8a8_dot<1>), grid, block, 0, stream, xq, x_scale, M, K, wq, w_scale, N, y, dbg);
  else if (M <= kGemvMaxM)
    hipLaunchKernelGGL((k_w8a8_dot<2>), grid, block, 0, stream, xq, x_scale, M, K, wq, w_scale, N, y, dbg);
  else if (M <= 16)
    hipLaunchKernelGGL((k_w8a8_mfma<1>), grid, block, 0, stream, xq, x_scale, M, K, wq, w_scale, N, y, dbg);
  else
    hipLaunchKernelGGL((k_w8a8_mfma<2>), grid, block, 0, stream, xq, x_scale, M, K, wq, w_scale, N, y, dbg);
  return hipGetLastError();
}
