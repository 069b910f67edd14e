// Persistent streaming driver shared by the linear kernels.
//
// A workgroup of WAVES waves walks the 16-row weight tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ... .  Inside a tile the K chunks are split into
// WAVES contiguous ranges of `per` chunks, one per wave, so every wave streams
// consecutive KiB of its tile.  The policy P supplies
//
//   typename P::template Batch<U>       registers of U chunks of loads
//   p.load<U>(batch, tile, j0, valid)   issue the loads of chunks j0..j0+U-1
//                                       (valid == false: zeros, no traffic)
//   p.compute<U>(batch, tile, j0)       consume them into the accumulators
//   p.finish(tile)                      reduce the waves' accumulators through
//                                       LDS, store the tile's outputs, reset
//                                       (contains __syncthreads)
//
// PIPE: the loads of the next batch -- including the first batch of the
// workgroup's next tile -- are issued before the current batch is consumed, so
// memory stays busy through the computation and across tile boundaries.  It
// needs every wave to own the same number of chunks, a multiple of 2*U.  The
// load/compute pairs are straight-line code (no branch between a load and its
// use), which keeps the compiler from sinking loads next to their uses, and
// scheduling barriers keep each batch's loads issued together.
#pragma once
#include "svg_device.h"

template <class P, int U>
SVG_DEV void stream_tiles_pipelined(P& p, int ntiles, int sb, int nbt) {
  using B = typename P::template Batch<U>;
  B A, Bt;
  int t = blockIdx.x;
  if (t >= ntiles) return;
  p.template load<U>(A, t, sb, true);
  for (; t < ntiles; t += gridDim.x) {
    const int tn = t + (int)gridDim.x;
    for (int q = 0; q < nbt; q += 2) {
      const int j = sb + q * U;
      p.template load<U>(Bt, t, j + U, true);
      __builtin_amdgcn_sched_barrier(0);
      p.template compute<U>(A, t, j);
      __builtin_amdgcn_sched_barrier(0);
      // next: the tile's next batch, else the first batch of the next tile
      const bool more = q + 2 < nbt;
      p.template load<U>(A, more ? t : tn, more ? j + 2 * U : sb, more || tn < ntiles);
      __builtin_amdgcn_sched_barrier(0);
      p.template compute<U>(Bt, t, j + U);
      __builtin_amdgcn_sched_barrier(0);
    }
    p.finish(t);
  }
}

template <class P>
SVG_DEV void stream_tiles_simple(P& p, int ntiles, int sb, int se) {
  using B = typename P::template Batch<1>;
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    for (int j = sb; j < se; ++j) {
      B A;
      p.template load<1>(A, t, j, true);
      p.template compute<1>(A, t, j);
    }
    p.finish(t);  // every wave joins, also one without chunks
  }
}
