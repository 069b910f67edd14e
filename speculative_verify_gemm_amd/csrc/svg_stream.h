// Persistent streaming kernel shared by the linear kernels (W4A8 and W8A8,
// dot-product and MFMA forms).
//
// A workgroup of WAVES waves walks the 16-row weight tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ... .  Every tile is cut along K into chunks (one
// KiB of weight codes each); wave w owns chunks [w*CPW, w*CPW + CPW) of every
// tile it visits, so
//
//  * its activation operands are the same for every tile: they are loaded
//    once, when the workgroup starts, and stay in registers -- only weight
//    codes and group parameters stream from HBM afterwards;
//  * the waves' partial sums of a tile are reduced through LDS in a fixed
//    order (deterministic), then scaled and stored.
//
// Weight loads run one batch of U chunks ahead of the computation, across tile
// boundaries too, so a wave keeps two batches in flight at all times; with
// U == CPW a tile's whole share is requested at once.  The load/compute pairs
// are straight-line code and scheduling barriers keep each batch's loads
// issued together (the compiler would otherwise sink loads next to their uses).
// CPW == 0 selects a plain loop (one chunk at a time, activations re-read)
// for K ranges too long to keep in registers.
//
// Policy interface (P):
//   P::kChunkK, P::kActRegs          k per chunk; activation VGPRs per chunk
//   P::red_t, P::kRedRows            LDS reduction element and rows per wave
//   typename P::template Acts<NC>    activation operands of NC chunks
//   typename P::template Batch<U>    weight codes and group parameters of U chunks
//   p.init(args, red)                per-thread set-up
//   p.load_acts<NC>(acts, j0)        chunks j0.. (chunks past K read zeros)
//   p.load<U>(batch, t, j0, valid)   issue the loads of chunks j0..j0+U-1 of tile t
//   p.compute<U, XI>(batch, acts, t, j0)   consume them with acts chunks XI..
//   p.finish(t, slot)                reduce through LDS buffer `slot`, store, reset
#pragma once
#include <algorithm>

#include "svg_device.h"
#include "svg_internal.h"

constexpr int kTileRows = 16;  // output rows per tile

struct LinArgs {
  const int8_t* xq;
  const float* x_scale;
  int M, K;
  const void* wq;
  const uint16_t* w_scale;
  const void* w_zero;
  int N;
  float* y;
  int32_t* dbg;
};

// Step Q of a tile: issue the next batch's loads (the tile's batch Q+1, or the
// first batch of the next tile), then consume batch Q.  `cur` holds batch Q.
template <class P, int CPW, int U, int Q>
struct TileSteps {
  template <class B, class X>
  static SVG_DEV void run(P& p, B& cur, B& nxt, const X& acts, int t, int tn, int ntiles, int sb) {
    constexpr int NB = CPW / U;
    constexpr bool last = Q + 1 == NB;
    p.template load<U>(nxt, last ? tn : t, last ? sb : sb + (Q + 1) * U, !last || tn < ntiles);
    __builtin_amdgcn_sched_barrier(0);
    p.template compute<U, Q * U>(cur, acts, t, sb + Q * U);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!last) TileSteps<P, CPW, U, Q + 1>::run(p, nxt, cur, acts, t, tn, ntiles, sb);
  }
};

template <class P, int CPW, int U>
SVG_DEV void stream_tiles_resident(P& p, int ntiles) {
  static_assert(CPW % U == 0, "batches must tile a wave's chunks");
  constexpr int NB = CPW / U;
  using B = typename P::template Batch<U>;
  using Steps = TileSteps<P, CPW, U, 0>;
  int t = blockIdx.x;
  if (t >= ntiles) return;  // uniform over the workgroup
  const int sb = p.wave * CPW;
  typename P::template Acts<CPW> acts;
  p.template load_acts<CPW>(acts, sb);
  B b0, b1;
  p.template load<U>(b0, t, sb, true);
  // Two tiles per iteration: with an odd number of batches per tile the next
  // tile's first batch lands in the other buffer.
  for (;;) {
    int tn = t + (int)gridDim.x;
    Steps::run(p, b0, b1, acts, t, tn, ntiles, sb);
    p.finish(t, 0);
    if (tn >= ntiles) break;
    t = tn;
    tn = t + (int)gridDim.x;
    if constexpr (NB % 2 == 0) Steps::run(p, b0, b1, acts, t, tn, ntiles, sb);
    else Steps::run(p, b1, b0, acts, t, tn, ntiles, sb);
    p.finish(t, 1);
    if (tn >= ntiles) break;
    t = tn;
  }
}

template <class P>
SVG_DEV void stream_tiles_simple(P& p, int ntiles, int sb, int se) {
  int slot = 0;
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    for (int j = sb; j < se; ++j) {
      typename P::template Acts<1> acts;
      typename P::template Batch<1> b;
      p.template load_acts<1>(acts, j);
      p.template load<1>(b, t, j, true);
      p.template compute<1, 0>(b, acts, t, j);
    }
    p.finish(t, slot);  // every wave joins, also one without chunks
    slot ^= 1;
  }
}

template <class P, int WAVES, int CPW, int U>
__global__ __launch_bounds__(WAVES * 64) void k_linear(LinArgs a) {
  __shared__ typename P::red_t red[2 * WAVES * P::kRedRows * kTileRows];
  const int ntiles = (a.N + kTileRows - 1) / kTileRows;
  P p;
  p.template init<WAVES>(a, red);
  if constexpr (CPW > 0) {
    stream_tiles_resident<P, CPW, U>(p, ntiles);
  } else {
    const int KT = (a.K + P::kChunkK - 1) / P::kChunkK;
    const int per = (KT + WAVES - 1) / WAVES;
    const int sb = min(KT, p.wave * per);
    stream_tiles_simple<P>(p, ntiles, sb, min(KT, sb + per));
  }
}

// Workgroups resident on the device at once for a kernel (cached per kernel:
// its occupancy is fixed when it is built).
template <auto KERNEL>
int resident_blocks(int block) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, KERNEL, block, 0) != hipSuccess || v < 1) v = 1;
    per_cu = v;
  }
  return per_cu * svg_cu_count();
}

// Persistent grid: at most as many workgroups as fit at once, and the tiles
// spread evenly (every workgroup walks the same number of tiles, give or take
// one) so none is left with a tail of its own.
template <class P, int WAVES, int CPW, int U>
hipError_t launch_linear(const LinArgs& a, hipStream_t stream) {
  constexpr auto kernel = k_linear<P, WAVES, CPW, U>;
  const int ntiles = (a.N + kTileRows - 1) / kTileRows;
  const int cap = resident_blocks<kernel>(WAVES * 64);
  const int rounds = (ntiles + cap - 1) / cap;
  const int grid = std::max(1, (ntiles + rounds - 1) / rounds);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}

// Launch shape from the number of K chunks: the fewest waves per workgroup
// (8, else 16) whose registers hold the activation operands of all chunks,
// with batches as large as the register budget allows.  The budget estimate
// is kActRegs VGPRs per activation chunk, kBatchRegs per chunk of each of the
// two weight batches in flight, and kFixedRegs for everything else; it must
// stay within 128 VGPRs (two 8-wave or one 16-wave workgroup per CU, all waves
// resident), else 192 for an 8-wave or 168 for a 12-wave workgroup alone on
// its CU.  K ranges that
// fit no shape take the plain loop.
template <class P>
hipError_t launch_linear_auto(const LinArgs& a, hipStream_t stream) {
  const int KT = (a.K + P::kChunkK - 1) / P::kChunkK;
#define SVG_FITS(CPW, U, LIM) (P::kActRegs * (CPW) + 2 * (U) * P::kBatchRegs + P::kFixedRegs <= (LIM))
#define SVG_TRY(W, CPW, U, LIM) \
  if constexpr (SVG_FITS(CPW, U, LIM)) return launch_linear<P, W, CPW, U>(a, stream)
  if (KT <= 8) { SVG_TRY(8, 1, 1, 192); }
  if (KT <= 16) { SVG_TRY(8, 2, 2, 128); else SVG_TRY(8, 2, 1, 192); }
  if (KT <= 32) { SVG_TRY(8, 4, 4, 128); else SVG_TRY(8, 4, 2, 192); }
  if (KT <= 64) { SVG_TRY(16, 4, 4, 128); else SVG_TRY(16, 4, 2, 128); }
  if (KT <= 96) { SVG_TRY(16, 6, 2, 128); else SVG_TRY(12, 8, 2, 168); else SVG_TRY(16, 6, 1, 128); }
  if (KT <= 128) { SVG_TRY(16, 8, 4, 128); else SVG_TRY(16, 8, 2, 128); }
  if (KT <= 192) { SVG_TRY(16, 12, 4, 128); else SVG_TRY(16, 12, 2, 128); }
#undef SVG_TRY
#undef SVG_FITS
  return launch_linear<P, 8, 0, 1>(a, stream);
}
