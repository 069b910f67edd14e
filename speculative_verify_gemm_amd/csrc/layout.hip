// Conversions between the canonical row-major layouts of encoded weights and
// activation codes and the library's storage (tiled weights, slab activation
// codes; both described in include/svgemm.h).
//
// Canonical layouts (the plainest reading of "4-bit codes, one scale and zero
// per group; 8-bit codes, one scale per row; int8 activation rows" in
// "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling",
// section "How Uzu optimizes bytes and tokens per pass"):
//   W4 codes   [N][K/2] bytes, code k in the low nibble of byte k/2 if k is even
//   W4 scales  [N][K/g] fp16;  fp16 zeros [N][K/g];
//   4-bit zeros [N][ceil(K/g/2)] bytes, group j in the low nibble if j is even
//   W8 codes   [N][K] int8;  W8 scales [N] fp16
//   act codes  [M][K] int8
//
// Every kernel is a gather: one thread per output word (or value), reading
// the source positions the layout maps it from; padding of the tiled storage
// is written as 0.  Pure data movement, bandwidth-bound, run offline (weights)
// or once per test.
#include <stdint.h>

#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kLayoutThreads = 256;

SVG_DEV int w4_code(const uint8_t* rows, int N, int K, int n, int k) {
  if (n >= N || k >= K) return 0;
  return (rows[(size_t)n * (K / 2) + (k >> 1)] >> (4 * (k & 1))) & 0xF;
}

// tiled W4 word `idx` (4 bytes) from canonical codes: tile = idx / 256 (one
// KiB), piece p = 16b + r (16 bytes, row 16i + r), bytes 0..7 the 16 codes
// from 128j + 16b, bytes 8..15 those from 128j + 64 + 16b; byte t of a word
// over k0..k0+7 holds code k0+t (low nibble) and k0+t+4 (high nibble)
__global__ void k_w4_codes_import(const uint8_t* __restrict__ rows, int N, int K, int KT, size_t nwords,
                                  u32* __restrict__ wq) {
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (idx >= nwords) return;
  const size_t tile = idx >> 8;
  const int wi = (int)(idx & 255);
  const int i = (int)(tile / KT), j = (int)(tile % KT);
  const int p = wi >> 2, q0 = (wi & 3) * 4;  // piece and its byte offset 0, 4, 8 or 12
  const int b = p >> 4, r = p & 15, n = 16 * i + r;
  const int k0 = 128 * j + 64 * (q0 >> 3) + 16 * b + 8 * ((q0 & 7) >> 2);
  u32 word = 0;
  for (int t = 0; t < 4; ++t) {
    const u32 byte = (u32)w4_code(rows, N, K, n, k0 + t) | ((u32)w4_code(rows, N, K, n, k0 + t + 4) << 4);
    word |= byte << (8 * t);
  }
  wq[idx] = word;
}

// canonical byte (n, kb) from tiled codes
SVG_DEV int w4_tiled_code(const uint8_t* wq, int KT, int n, int k) {
  const int i = n >> 4, r = n & 15, j = k >> 7, kk = k & 127;
  const int half = kk >> 6, kin = kk & 63, b = kin >> 4, o = kin & 15;
  const int w = o >> 3, u = o & 7, t = u & 3, hi = u >> 2;
  const uint8_t byte = wq[((size_t)i * KT + j) * 1024 + (size_t)(16 * b + r) * 16 + half * 8 + w * 4 + t];
  return (byte >> (4 * hi)) & 0xF;
}

__global__ void k_w4_codes_export(const uint8_t* __restrict__ wq, int N, int K, int KT, uint8_t* __restrict__ rows) {
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  const size_t per_row = (size_t)K / 2;
  if (idx >= (size_t)N * per_row) return;
  const int n = (int)(idx / per_row), k = 2 * (int)(idx % per_row);
  rows[idx] = (uint8_t)(w4_tiled_code(wq, KT, n, k) | (w4_tiled_code(wq, KT, n, k + 1) << 4));
}

// Group parameters: tiled index v of value (n, g) is ((i*KB + jb)*16 + r)*GB + c
// with i = n/16, r = n%16, jb = g/GB, c = g%GB, GB = 512/group.
struct ParamMap {
  int N, NG, KB, GB;
  SVG_DEV void of(size_t v, int& n, int& g) const {
    const int c = (int)(v % GB);
    const size_t rest = v / GB;
    const int r = (int)(rest % 16);
    const size_t rest2 = rest / 16;
    const int jb = (int)(rest2 % KB), i = (int)(rest2 / KB);
    n = 16 * i + r;
    g = jb * GB + c;
  }
  SVG_DEV size_t at(int n, int g) const {
    return (((size_t)(n >> 4) * KB + g / GB) * 16 + (n & 15)) * GB + g % GB;
  }
  SVG_DEV bool real(int n, int g) const { return n < N && g < NG; }
};

__global__ void k_param16_import(const uint16_t* __restrict__ rows, ParamMap m, size_t nvals,
                                 uint16_t* __restrict__ out) {
  const size_t v = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (v >= nvals) return;
  int n, g;
  m.of(v, n, g);
  out[v] = m.real(n, g) ? rows[(size_t)n * m.NG + g] : (uint16_t)0;
}

__global__ void k_param16_export(const uint16_t* __restrict__ tiled, ParamMap m, uint16_t* __restrict__ rows) {
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (idx >= (size_t)m.N * m.NG) return;
  const int n = (int)(idx / m.NG), g = (int)(idx % m.NG);
  rows[idx] = tiled[m.at(n, g)];
}

SVG_DEV int z4_row_bytes(int NG) { return (NG + 1) / 2; }

// 4-bit zeros: tiled byte vb holds values 2vb (low nibble) and 2vb + 1
__global__ void k_z4_import(const uint8_t* __restrict__ rows, ParamMap m, size_t nbytes, uint8_t* __restrict__ out) {
  const size_t vb = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (vb >= nbytes) return;
  const int zs = z4_row_bytes(m.NG);
  u32 byte = 0;
  for (int h = 0; h < 2; ++h) {
    int n, g;
    m.of(2 * vb + h, n, g);
    if (m.real(n, g)) byte |= (u32)((rows[(size_t)n * zs + (g >> 1)] >> (4 * (g & 1))) & 0xF) << (4 * h);
  }
  out[vb] = (uint8_t)byte;
}

__global__ void k_z4_export(const uint8_t* __restrict__ tiled, ParamMap m, uint8_t* __restrict__ rows) {
  const int zs = z4_row_bytes(m.NG);
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (idx >= (size_t)m.N * zs) return;
  const int n = (int)(idx / zs), zb = (int)(idx % zs);
  u32 byte = 0;
  for (int h = 0; h < 2; ++h) {
    const int g = 2 * zb + h;
    if (g >= m.NG) break;
    const size_t v = m.at(n, g);
    byte |= (u32)((tiled[v >> 1] >> (4 * (v & 1))) & 0xF) << (4 * h);
  }
  rows[idx] = (uint8_t)byte;
}

// W8 tile (i, j): 16 rows x 64 k, piece 16b + r = row 16i + r, k in
// [64j + 16b, +16) in natural order
__global__ void k_w8_codes_import(const int8_t* __restrict__ rows, int N, int K, int KT8, size_t nwords,
                                  u32* __restrict__ wq) {
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (idx >= nwords) return;
  const size_t tile = idx >> 8;
  const int wi = (int)(idx & 255);
  const int i = (int)(tile / KT8), j = (int)(tile % KT8);
  const int p = wi >> 2, o0 = (wi & 3) * 4;
  const int b = p >> 4, r = p & 15, n = 16 * i + r;
  const int k0 = 64 * j + 16 * b + o0;
  u32 word = 0;
  for (int t = 0; t < 4; ++t) {
    const int k = k0 + t;
    const u32 c = (n < N && k < K) ? (u32)(uint8_t)rows[(size_t)n * K + k] : 0u;
    word |= c << (8 * t);
  }
  wq[idx] = word;
}

__global__ void k_w8_codes_export(const int8_t* __restrict__ wq, int N, int K, int KT8, int8_t* __restrict__ rows) {
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (idx >= (size_t)N * K) return;
  const int n = (int)(idx / K), k = (int)(idx % K);
  const int i = n >> 4, r = n & 15, j = k >> 6, kk = k & 63, b = kk >> 4, o = kk & 15;
  rows[idx] = wq[((size_t)i * KT8 + j) * 1024 + (size_t)(16 * b + r) * 16 + o];
}

__global__ void k_copy16(const uint16_t* __restrict__ src, size_t n, uint16_t* __restrict__ dst) {
  const size_t idx = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;
  if (idx < n) dst[idx] = src[idx];
}

// Activation codes, 4 bytes per thread: slab byte (m, k) sits at
// ((k/32)*M + m)*32 + k%32.
__global__ void k_act_to_slab(const u32* __restrict__ rows, int M, int K, u32* __restrict__ slab) {
  const size_t w = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;  // slab word
  if (w >= (size_t)M * K / 4) return;
  const size_t s = w / (8 * (size_t)M), rem = w % (8 * (size_t)M);
  const int m = (int)(rem / 8), kw = (int)(rem % 8);
  slab[w] = rows[((size_t)m * K + s * 32) / 4 + kw];
}

__global__ void k_act_from_slab(const u32* __restrict__ slab, int M, int K, u32* __restrict__ rows) {
  const size_t w = (size_t)blockIdx.x * kLayoutThreads + threadIdx.x;  // row word
  if (w >= (size_t)M * K / 4) return;
  const int m = (int)(w / (K / 4)), k = (int)(w % (K / 4)) * 4;
  rows[w] = slab[(((size_t)(k / 32) * M + m) * 32 + (k & 31)) / 4];
}

dim3 grid_for(size_t n) { return dim3((unsigned)((n + kLayoutThreads - 1) / kLayoutThreads)); }

}  // namespace

hipError_t svg_launch_import_weights(int fmt_w8, int z4, int group, int N, int K, const void* codes,
                                     const uint16_t* scale, const void* zero, void* wq, uint16_t* w_scale,
                                     void* w_zero, hipStream_t stream) {
  if (fmt_w8) {
    const int KT8 = (K + 63) / 64;
    const size_t nwords = (size_t)(N + 15) / 16 * 16 * KT8 * 64 / 4;
    hipLaunchKernelGGL(k_w8_codes_import, grid_for(nwords), dim3(kLayoutThreads), 0, stream,
                       static_cast<const int8_t*>(codes), N, K, KT8, nwords, static_cast<u32*>(wq));
    hipLaunchKernelGGL(k_copy16, grid_for((size_t)N), dim3(kLayoutThreads), 0, stream, scale, (size_t)N, w_scale);
    return hipGetLastError();
  }
  const int KT = (K + 127) / 128;
  const size_t Np = (size_t)(N + 15) / 16 * 16;
  const size_t nwords = Np * KT * 64 / 4;
  hipLaunchKernelGGL(k_w4_codes_import, grid_for(nwords), dim3(kLayoutThreads), 0, stream,
                     static_cast<const uint8_t*>(codes), N, K, KT, nwords, static_cast<u32*>(wq));
  const ParamMap m{N, K / group, (K + kMetaK - 1) / kMetaK, kMetaK / group};
  const size_t nvals = Np * m.KB * m.GB;
  hipLaunchKernelGGL(k_param16_import, grid_for(nvals), dim3(kLayoutThreads), 0, stream, scale, m, nvals, w_scale);
  if (z4)
    hipLaunchKernelGGL(k_z4_import, grid_for(nvals / 2), dim3(kLayoutThreads), 0, stream,
                       static_cast<const uint8_t*>(zero), m, nvals / 2, static_cast<uint8_t*>(w_zero));
  else
    hipLaunchKernelGGL(k_param16_import, grid_for(nvals), dim3(kLayoutThreads), 0, stream,
                       static_cast<const uint16_t*>(zero), m, nvals, static_cast<uint16_t*>(w_zero));
  return hipGetLastError();
}

hipError_t svg_launch_export_weights(int fmt_w8, int z4, int group, int N, int K, const void* wq,
                                     const uint16_t* w_scale, const void* w_zero, void* codes, uint16_t* scale,
                                     void* zero, hipStream_t stream) {
  if (fmt_w8) {
    const int KT8 = (K + 63) / 64;
    hipLaunchKernelGGL(k_w8_codes_export, grid_for((size_t)N * K), dim3(kLayoutThreads), 0, stream,
                       static_cast<const int8_t*>(wq), N, K, KT8, static_cast<int8_t*>(codes));
    hipLaunchKernelGGL(k_copy16, grid_for((size_t)N), dim3(kLayoutThreads), 0, stream, w_scale, (size_t)N, scale);
    return hipGetLastError();
  }
  const int KT = (K + 127) / 128;
  hipLaunchKernelGGL(k_w4_codes_export, grid_for((size_t)N * K / 2), dim3(kLayoutThreads), 0, stream,
                     static_cast<const uint8_t*>(wq), N, K, KT, static_cast<uint8_t*>(codes));
  const ParamMap m{N, K / group, (K + kMetaK - 1) / kMetaK, kMetaK / group};
  hipLaunchKernelGGL(k_param16_export, grid_for((size_t)N * m.NG), dim3(kLayoutThreads), 0, stream, w_scale, m,
                     scale);
  if (z4)
    hipLaunchKernelGGL(k_z4_export, grid_for((size_t)N * ((m.NG + 1) / 2)), dim3(kLayoutThreads), 0, stream,
                       static_cast<const uint8_t*>(w_zero), m, static_cast<uint8_t*>(zero));
  else
    hipLaunchKernelGGL(k_param16_export, grid_for((size_t)N * m.NG), dim3(kLayoutThreads), 0, stream,
                       static_cast<const uint16_t*>(w_zero), m, static_cast<uint16_t*>(zero));
  return hipGetLastError();
}

hipError_t svg_launch_act_codes(int to_slab, const int8_t* src, int M, int K, int8_t* dst, hipStream_t stream) {
  const size_t nwords = (size_t)M * K / 4;
  if (to_slab)
    hipLaunchKernelGGL(k_act_to_slab, grid_for(nwords), dim3(kLayoutThreads), 0, stream,
                       reinterpret_cast<const u32*>(src), M, K, reinterpret_cast<u32*>(dst));
  else
    hipLaunchKernelGGL(k_act_from_slab, grid_for(nwords), dim3(kLayoutThreads), 0, stream,
                       reinterpret_cast<const u32*>(src), M, K, reinterpret_cast<u32*>(dst));
  return hipGetLastError();
}
