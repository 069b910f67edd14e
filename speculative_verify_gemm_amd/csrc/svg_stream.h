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
#include <atomic>
#include <type_traits>

#include "svg_act.h"
#include "svg_device.h"
#include "svg_internal.h"

constexpr int kTileRows = 16;  // output rows per tile

// xq: activation codes in 32-k slabs (include/svgemm.h): byte (m, k) of a
// buffer of ldm rows at ((k / 32) * ldm + m) * 32 + k % 32.  A launch covers
// rows m0 .. m0 + M - 1 of it (x_scale, y and dbg already point at row m0).
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
  int ldm, m0;
};

// Byte offset of the 16 codes k0 .. k0 + 15 (k0 % 16 == 0) of row m.
SVG_DEV u32 act_slab_off(int m, int k0, int ldm) {
  return ((u32)(k0 >> 5) * (u32)ldm + (u32)m) * 32u + (u32)(k0 & 31);
}

// Step Q of a tile: issue the next batch's loads (the tile's batch Q+1, or the
// first batch of the next tile), then consume batch Q.  `cur` holds batch Q.
// SKIP0: the loads of step 0 were issued earlier (see stream_tiles_resident).
template <class P, int CPW, int U, int Q, bool SKIP0 = false>
struct TileSteps {
  template <class B>
  static SVG_DEV void issue_next(P& p, B& nxt, int t, int tn, int ntiles, int sb) {
    constexpr bool last = Q + 1 == CPW / U;
    p.template load<U>(nxt, last ? tn : t, last ? sb : sb + (Q + 1) * U, !last || tn < ntiles);
  }
  template <class B, class X>
  static SVG_DEV void run(P& p, B& cur, B& nxt, const X& acts, int t, int tn, int ntiles, int sb) {
    constexpr bool last = Q + 1 == CPW / U;
    if constexpr (!(SKIP0 && Q == 0)) issue_next(p, nxt, t, tn, ntiles, sb);
    __builtin_amdgcn_sched_barrier(0);
    p.template compute<U, Q * U>(cur, acts, t, sb + Q * U);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!last) TileSteps<P, CPW, U, Q + 1>::run(p, nxt, cur, acts, t, tn, ntiles, sb);
  }
};

// The workgroup walks tiles first, first + stride, ...  `pre()` runs before
// the first weight batch is requested and `gate()` after it, before the
// activations are read (the fused kernel quantizes its input rows there).  With LDS, the
// activation operands come from the workgroup's own LDS copy of the quantized
// rows (P::load_acts<NC, true>) instead of global memory, and the second batch
// is requested before the gate too, so that two batches stream while the
// rows are being quantized.  (With global activations the second batch waits:
// loads complete in order, so activations requested after it would hold the
// first computation back.)
template <class P, int CPW, int U, bool LDS, int AUX, class Pre, class Gate>
SVG_DEV void stream_tiles_resident(P& p, int ntiles, int first, int stride, Pre&& pre, Gate&& gate) {
  static_assert(CPW % U == 0, "batches must tile a wave's chunks");
  constexpr int NB = CPW / U;
  using B = typename P::template Batch<U>;
  using Steps = TileSteps<P, CPW, U, 0>;
  int t = first;
  if (t >= ntiles) return;  // uniform over the workgroup
  const int sb = p.wave * CPW;
  int tn = t + stride;
  B b0, b1;
  pre();
  __builtin_amdgcn_sched_barrier(0);
  p.template load<U>(b0, t, sb, true);
  if constexpr (LDS) Steps::issue_next(p, b1, t, tn, ntiles, sb);
  __builtin_amdgcn_sched_barrier(0);
  gate();
  typename P::template Acts<CPW> acts;
  p.template load_acts<CPW, LDS, AUX>(acts, sb);
  TileSteps<P, CPW, U, 0, LDS>::run(p, b0, b1, acts, t, tn, ntiles, sb);
  p.finish(t, 0);
  // Two tiles per iteration: with an odd number of batches per tile the next
  // tile's first batch lands in the other buffer.
  for (;;) {
    if (tn >= ntiles) break;
    t = tn;
    tn = t + stride;
    if constexpr (NB % 2 == 0) Steps::run(p, b0, b1, acts, t, tn, ntiles, sb);
    else Steps::run(p, b1, b0, acts, t, tn, ntiles, sb);
    p.finish(t, 1);
    if (tn >= ntiles) break;
    t = tn;
    tn = t + stride;
    Steps::run(p, b0, b1, acts, t, tn, ntiles, sb);
    p.finish(t, 0);
  }
}

template <class P, bool LDS, int AUX>
SVG_DEV void stream_tiles_simple(P& p, int ntiles, int first, int stride, int sb, int se) {
  int slot = 0;
  for (int t = first; t < ntiles; t += stride) {
    for (int j = sb; j < se; ++j) {
      typename P::template Acts<1> acts;
      typename P::template Batch<1> b;
      p.template load_acts<1, LDS, AUX>(acts, j);
      p.template load<1>(b, t, j, true);
      p.template compute<1, 0>(b, acts, t, j);
    }
    p.finish(t, slot);  // every wave joins, also one without chunks
    slot ^= 1;
  }
}

// AUX: cache policy of the activation loads from global memory
template <class P, int WAVES, int CPW, int U, bool LDS = false, int AUX = 0, class Pre, class Gate>
SVG_DEV void stream_tiles(P& p, const LinArgs& a, int first, int stride, Pre&& pre, Gate&& gate) {
  const int ntiles = (a.N + kTileRows - 1) / kTileRows;
  if constexpr (CPW > 0) {
    stream_tiles_resident<P, CPW, U, LDS, AUX>(p, ntiles, first, stride, pre, gate);
  } else {
    if (first >= ntiles) return;
    pre();
    gate();
    const int KT = (a.K + P::kChunkK - 1) / P::kChunkK;
    const int per = (KT + WAVES - 1) / WAVES;
    const int sb = min(KT, p.wave * per);
    stream_tiles_simple<P, LDS, AUX>(p, ntiles, first, stride, sb, min(KT, sb + per));
  }
}

// All kernel arguments fetched in one round trip.  Left alone, the compiler
// requests N first (for a workgroup's early exit when it has no tile), waits,
// and only then requests the rest -- two or three dependent kernel-argument
// loads ahead of the first weight request (measured: the first request
// 0.2 us later, launches 0.1-0.3 us longer).  Taking every value into scalar
// registers here puts all the loads ahead of a single wait.
SVG_DEV void args_at_once(const LinArgs& a) {
  asm volatile("" ::"s"(a.xq), "s"(a.x_scale), "s"(a.M), "s"(a.K), "s"(a.wq), "s"(a.w_scale), "s"(a.w_zero),
               "s"(a.N), "s"(a.y), "s"(a.dbg), "s"(a.ldm), "s"(a.m0));
}

template <class P, int WAVES, int CPW, int U>
__global__ __launch_bounds__(WAVES * 64) void k_linear(LinArgs a) {
  __shared__ typename P::red_t red[2 * WAVES * P::kRedRows * kTileRows];
  args_at_once(a);
  P p;
  p.template init<WAVES>(a, red);
  stream_tiles<P, WAVES, CPW, U>(p, a, blockIdx.x, gridDim.x, [] {}, [] {});
}

// ------------------------------------------------------ fused activation input
// The fused kernel takes the fp32 activation rows X of a GEMV-sized call
// (M <= fused_rows<P>(): the GEMV policies' one or two rows), and every
// workgroup rotates and quantizes them itself into LDS while its first two
// weight batches are in flight, then reads its activation operands from
// there: no launch of its own for the quantization and nothing shared between
// workgroups.  Workgroup 0 also writes xq and x_scale (the values
// act_rht_quant_i8 gives).  K <= kLdsMaxK.
//
// The MFMA policies are not fused: measured at M = 2..4, first with whole
// rows quantized by the whole workgroup (6 to 10 us per launch against 4 to
// 6 us for a launch of its own), then with each wave quantizing its own
// stretch of every row (the g128 stack's M = 2 and 4 passes 10 and 15 %
// slower than with the quantization launch: the rows' registers leave one
// workgroup per CU).  Publishing the rows from M workgroups to the others inside one
// launch (k_linear_shared below) works but was measured slower than the
// quantization launch too: at M = 16, K = 4096 the publishers are done about
// 2.8 us after the launch starts and the readers see the last row about 5 us
// in, a hand-off that costs more than a launch boundary.
constexpr int kLdsMaxK = 12288;
template <class P>
constexpr int fused_rows() { return P::kFusedRows; }

struct ActIn {
  const float* X;
  const int8_t* signs;
  int block;          // transform block, 32 or 64
  u32* ws = nullptr;  // the launch's workspace for shared quantization (k_linear_shared), if any
};

template <class P, int WAVES, int CPW, int U>
__global__ __launch_bounds__(WAVES * 64) void k_linear_fused(LinArgs a, ActIn f) {
  constexpr int R = fused_rows<P>();  // LDS rows
  static_assert(R > 0, "only the GEMV policies are fused");
  args_at_once(a);
  asm volatile("" ::"s"(f.X), "s"(f.signs), "s"(f.block));
  // How the row(s) get quantized.
  //  * On the resident walk (kOwn): every wave requests just the part of each
  //    row its own chunks cover (OWN_V values from k = wave * OWN_V) before
  //    its weights, rotates it, joins one workgroup-wide maximum per row, and
  //    writes its codes to its own stretch of the LDS rows (row stride: all
  //    waves' stretches), from which it reads its operands back -- no barrier
  //    between codes and operands, since no other wave reads that stretch.
  //  * Otherwise (the plain walk, or shapes wider than LDS): one row is held by as many
  //    leading waves as hold it with kLoadCPT chunks per lane, requested
  //    before their weights while the other waves request weights first
  //    (row_early); two rows, or a row too long for that, are quantized by
  //    the whole workgroup after its first weight batches (CPT chunks per
  //    thread per row in registers: enough for every K the resident shapes of
  //    this size take -- K <= 4096 with 8 waves, <= 12288 with 12 or 16 --
  //    and longer rows one at a time).  The codes go to the shared LDS rows
  //    (zero-padded) and a barrier precedes the operand reads.
  constexpr bool kOwn = CPW > 0 && WAVES * CPW * P::kChunkK <= kLdsMaxK;
  constexpr int OWN_V = CPW * P::kChunkK;                    // values per wave
  constexpr int OWN_CPT = kOwn ? (OWN_V / 4 + 63) / 64 : 1;  // float4 chunks per lane
  constexpr int OWN_ROW = WAVES * OWN_V / 4;                 // LDS words per row
  constexpr int CPT = WAVES >= 16 ? 3 : (WAVES >= 12 ? 4 : 2);
  constexpr int kLoadCPT = 4;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  const int own_k0 = wave * OWN_V;
  const int own_k = kOwn ? max(0, min(OWN_V, a.K - own_k0)) : 0;  // real values of this wave's part
  const int nchunk = a.K >> 2;
  const int LT = min((int)blockDim.x, (nchunk + 64 * kLoadCPT - 1) / (64 * kLoadCPT) * 64);
  const bool row_early = !kOwn && R == 1 && nchunk <= LT * kLoadCPT;
  RowRegs<OWN_CPT> own[R];
  RowRegs<kLoadCPT> early;
  __shared__ typename P::red_t red[2 * WAVES * P::kRedRows * kTileRows];
  __shared__ float act_red[16 * R];
  __shared__ __align__(16) u32 xl[R * kLdsMaxK / 4];
  __shared__ float xsl[R];
  __shared__ float own_scale[WAVES * R];  // each wave's copy of the row scales (wave 0's is xsl)
  P p;
  p.template init<WAVES>(a, red);
  const int KP = ((a.K + 127) >> 7) * 32;  // words per LDS row: K padded to whole 128-k chunks
  stream_tiles<P, WAVES, CPW, U, true>(p, a, blockIdx.x, gridDim.x, [&] {
    if constexpr (kOwn) {
      // past its real values a part reads zeros (the resource ends there);
      // rows past M read nothing
#pragma unroll
      for (int m = 0; m < R; ++m)
        act_load_row<OWN_CPT>(f.X + (size_t)m * a.K + own_k0, m < a.M ? own_k : 0, f.signs + own_k0, own[m],
                              (u32)lane, 64u);
    } else {
      if (row_early && (int)threadIdx.x < LT) act_load_row<kLoadCPT>(f.X, a.K, f.signs, early, threadIdx.x, LT);
    }
  }, [&] {
    // the transform block is uniform over the launch: both forms are in the
    // kernel and one branch picks
    if constexpr (kOwn) {
      auto quantize = [&](auto block) {
        constexpr int B = decltype(block)::value;
        float amax[R];
#pragma unroll
        for (int m = 0; m < R; ++m) amax[m] = act_rotate_loaded<OWN_CPT, B>(own[m]);
        if constexpr (R == 1) amax[0] = wg_max_once(amax[0], act_red);
        else wg_max_rows<R>(amax, act_red);
#pragma unroll
        for (int m = 0; m < R; ++m) {
          u32* wl = xl + m * OWN_ROW + own_k0 / 4;
          const int real = m < a.M ? own_k : 0;
          if (real > 0)
            act_store_codes<OWN_CPT, StoreLds, B>(own[m], real, amax[m],
                                                  StoreLds{wl, wave == 0 ? xsl + m : own_scale + wave * R + m},
                                                  (u32)lane, 64u);
          for (int c = real / 4 + lane; c < OWN_V / 4; c += 64) wl[c] = 0u;  // k past K, rows past M
        }
      };
      if (f.block == 64) quantize(std::integral_constant<int, 64>{});
      else quantize(std::integral_constant<int, 32>{});
      if (blockIdx.x == 0) {  // the call's xq / x_scale outputs, each wave its part
        for (int m = 0; m < a.M; ++m)
          for (int c = lane; c < own_k / 4; c += 64) {
            const int w = own_k0 / 4 + c;  // word w (k = 4w) of row m
            reinterpret_cast<u32*>(const_cast<int8_t*>(a.xq))[((w >> 3) * a.ldm + a.m0 + m) * 8 + (w & 7)] =
                xl[m * OWN_ROW + w];
          }
        if (threadIdx.x == 0)
          for (int m = 0; m < a.M; ++m) const_cast<float*>(a.x_scale)[m] = xsl[m];
      }
      // the operand reads below must follow this wave's own LDS writes
      asm volatile("" ::: "memory");
    } else {
      for (int i = threadIdx.x; i < R * KP; i += blockDim.x)  // zero the padding (rows past M, k past K)
        if (i / KP >= a.M || (i % KP) * 4 >= a.K) xl[i] = 0u;
      auto quantize = [&](auto block) {
        constexpr int B = decltype(block)::value;
        if (row_early) {
          const bool holds = (int)threadIdx.x < LT;
          const float amax = wg_max_once(holds ? act_rotate_loaded<kLoadCPT, B>(early) : 0.f, act_red);
          if (holds)
            act_store_codes<kLoadCPT, StoreLds, B>(early, a.K, amax, StoreLds{xl, xsl}, threadIdx.x, LT);
        } else if (a.K <= 4 * CPT * (int)blockDim.x) {
          act_quant_rows_lds<R, CPT, B>(f.X, a.M, a.K, f.signs, xl, KP, xsl, act_red);
        } else {
          for (int m = 0; m < a.M; ++m)
            act_quant_row<CPT, StoreLds, B>(f.X + (size_t)m * a.K, a.K, f.signs,
                                            StoreLds{xl + m * KP, xsl + m}, act_red);
        }
      };
      if (f.block == 64) quantize(std::integral_constant<int, 64>{});
      else quantize(std::integral_constant<int, 32>{});
      __syncthreads();
      if (blockIdx.x == 0) {  // the call's xq / x_scale outputs
        for (int i = threadIdx.x; i < a.M * (a.K / 4); i += blockDim.x) {
          const int m = i / (a.K / 4), w = i % (a.K / 4);  // word w (k = 4w) of row m
          reinterpret_cast<u32*>(const_cast<int8_t*>(a.xq))[((w >> 3) * a.ldm + a.m0 + m) * 8 + (w & 7)] =
              xl[m * KP + w];
        }
        if (threadIdx.x < a.M) const_cast<float*>(a.x_scale)[threadIdx.x] = xsl[threadIdx.x];
      }
    }
    p.xlds = reinterpret_cast<const int8_t*>(xl);
    p.xlds_row = (kOwn ? OWN_ROW : KP) * 4;
    p.x_scale = xsl;
  });
}

// ------------------------------------------------- shared activation input
// The rows of a verify batch (M >= 2, or a row too long for the fused
// kernel's LDS), quantized once per launch instead of in a launch of their
// own: workgroup m (m < M) rotates and quantizes row m into xq / x_scale and
// counts it in; every workgroup waits until all M rows are in before it
// reads its activation operands.  The last workgroup to finish zero-fills the
// counters for the next call.  Workspace words (zero-filled before first
// use): 1 rows counted in, 2 workgroups finished, 3 give-up flag (sticky: set
// if the bounded wait ran out; then y is undefined).
template <class P, int WAVES, int CPW, int U>
__global__ __launch_bounds__(WAVES * 64) void k_linear_shared(LinArgs a, ActIn f) {
  constexpr int CPT = WAVES >= 16 ? 3 : (WAVES >= 12 ? 4 : 2);
  args_at_once(a);
  asm volatile("" ::"s"(f.X), "s"(f.signs), "s"(f.block), "s"(f.ws));
  __shared__ typename P::red_t red[2 * WAVES * P::kRedRows * kTileRows];
  __shared__ float act_red[16];
  __shared__ float xsl[P::kMaxTok];
  P p;
  p.template init<WAVES>(a, red);
  u32* ws = f.ws;
  // Coherence across XCCs without cache maintenance: the publishers write the
  // codes and scales through to memory (sc1 stores, then a wait for their
  // acknowledgement) before counting them in; readers load them with sc1
  // loads, which bypass the XCC's L2 -- a line of xq cached there by an
  // earlier call would otherwise be read stale.
  // Publishers are the workgroups with the lowest indices: workgroups are
  // dispatched in index order, so a running workgroup's publishers have been
  // dispatched too (running or done) -- no wait depends on one that is not.
  // A publisher quantizes before it requests any weights; every workgroup
  // requests its first weight batch before it waits for the rows, so that
  // batch streams in meanwhile.
  const int G = gridDim.x, bid = blockIdx.x;
  stream_tiles<P, WAVES, CPW, U, false, kSC1>(p, a, bid, G, [&] {
    if (bid < a.M) {
      auto quantize = [&](auto block) {
        constexpr int B = decltype(block)::value;
        for (int m = bid; m < a.M; m += G)
          act_quant_row<CPT, StoreGlobalT<kSC1>, B>(f.X + (size_t)m * a.K, a.K, f.signs,
                                                    StoreGlobalT<kSC1>(const_cast<int8_t*>(a.xq), a.m0 + m, a.ldm,
                                                                       const_cast<float*>(a.x_scale) + m, a.K),
                                                    act_red);
      };
      if (f.block == 64) quantize(std::integral_constant<int, 64>{});
      else quantize(std::integral_constant<int, 32>{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's codes and scale are performed
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(ws + 1, (u32)((a.M - bid + G - 1) / G), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }, [&] {
    if (threadIdx.x == 0) {
      for (u32 it = 0; __hip_atomic_load(ws + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (u32)a.M; ++it) {
        if (it > (1u << 20)) {  // about a second of device-scope polls: give up rather than hang
          __hip_atomic_store(ws + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < a.M && (int)threadIdx.x < P::kMaxTok)
      xsl[threadIdx.x] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          make_rsrc(a.x_scale, (u32)a.M * 4u), threadIdx.x * 4u, 0, kSC1));
    __syncthreads();
    p.x_scale = xsl;
  });
  __syncthreads();
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(ws + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
    __hip_atomic_store(ws + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ws + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups resident on the device at once for a kernel (cached per kernel:
// its occupancy is fixed when it is built).
template <auto KERNEL>
int resident_blocks(int block) {
  static std::atomic<int> per_cu{0};  // every calling thread finds the same value
  int v = per_cu.load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, KERNEL, block, 0) != hipSuccess || v < 1) v = 1;
    per_cu.store(v, std::memory_order_relaxed);
  }
  return v * svg_cu_count();
}

// Persistent grid: at most as many workgroups as fit at once, and the tiles
// spread evenly (every workgroup walks the same number of tiles, give or take
// one) so none is left with a tail of its own.  Then per compute unit: the
// busiest CU holds ceil(G / CUs) workgroups of ceil(tiles / G) tiles each,
// and a CU running two workgroups streams barely faster than one (measured:
// 768 tiles of 16 x 4096 W4 on 384 workgroups end about 1 us later than on
// 256, where every CU walks 3 tiles instead of 4 on half of them), so a grid
// of whole CU multiples replaces it where that busiest CU gets fewer tiles.
template <auto KERNEL>
int spread_grid(int ntiles, int block) {
  const int cap = resident_blocks<KERNEL>(block);
  const int rounds = (ntiles + cap - 1) / cap;
  int G = std::max(1, (ntiles + rounds - 1) / rounds);
  const int ncu = svg_cu_count();
  auto busiest = [&](int g) { return ((g + ncu - 1) / ncu) * ((ntiles + g - 1) / g); };
  int load = busiest(G);
  for (int g = ncu; g <= std::min(cap, ntiles); g += ncu)
    if (busiest(g) < load) { load = busiest(g); G = g; }
  return G;
}

// f != nullptr: the input rows are fp32.  Calls of at most fused_rows<P>()
// rows take the fused kernel; otherwise, with a workspace, the shared kernel;
// else the rows are quantized in a launch of their own first.
template <class P, int WAVES, int CPW, int U>
hipError_t launch_linear(const LinArgs& a, const ActIn* f, hipStream_t stream) {
  const int ntiles = (a.N + kTileRows - 1) / kTileRows;
  if (f) {
    if constexpr (fused_rows<P>() > 0) {
      if (a.M <= fused_rows<P>() && a.K <= kLdsMaxK) {
        constexpr auto kernel = k_linear_fused<P, WAVES, CPW, U>;
        hipLaunchKernelGGL(kernel, dim3(spread_grid<kernel>(ntiles, WAVES * 64)), dim3(WAVES * 64), 0, stream,
                           a, *f);
        return hipGetLastError();
      }
    }
    if (f->ws) {
      constexpr auto kernel = k_linear_shared<P, WAVES, CPW, U>;
      hipLaunchKernelGGL(kernel, dim3(spread_grid<kernel>(ntiles, WAVES * 64)), dim3(WAVES * 64), 0, stream,
                         a, *f);
      return hipGetLastError();
    }
    hipError_t e = svg_launch_act_rht_quant(f->X, a.M, a.K, f->signs, f->block, const_cast<int8_t*>(a.xq),
                                            const_cast<float*>(a.x_scale), stream);
    if (e != hipSuccess) return e;
  }
  {
    constexpr auto kernel = k_linear<P, WAVES, CPW, U>;
    hipLaunchKernelGGL(kernel, dim3(spread_grid<kernel>(ntiles, WAVES * 64)), dim3(WAVES * 64), 0, stream, a);
  }
  return hipGetLastError();
}

// Launch shape from the number of K chunks: the fewest waves per workgroup
// (8, else 16) whose registers hold the activation operands of all chunks,
// with batches as large as the register budget allows.  The budget estimate
// is kActRegs VGPRs per activation chunk, kBatchRegs per chunk of each of the
// two weight batches in flight, and kFixedRegs for everything else; it must
// stay within 128 VGPRs (two 8-wave or one 16-wave workgroup per CU, all waves
// resident), else 192 for an 8-wave or 168 for a 12-wave workgroup alone on
// its CU, and last 256 (an 8-wave workgroup alone on its CU, two waves per
// SIMD: the 16 or 32 token rows of K = 12288 stay resident that way, which
// halves the launch time against the plain loop).  K ranges that fit no
// shape take the plain loop.
template <class P>
hipError_t launch_linear_auto(const LinArgs& a, const ActIn* f, hipStream_t stream) {
  const int KT = (a.K + P::kChunkK - 1) / P::kChunkK;
#define SVG_FITS(CPW, U, LIM) (P::kActRegs * (CPW) + 2 * (U) * P::kBatchRegs + P::kFixedRegs <= (LIM))
#define SVG_TRY(W, CPW, U, LIM) \
  if constexpr (SVG_FITS(CPW, U, LIM)) return launch_linear<P, W, CPW, U>(a, f, stream)
  if (KT <= 8) { SVG_TRY(8, 1, 1, 192); }
  if (KT <= 16) { SVG_TRY(8, 2, 2, 128); else SVG_TRY(8, 2, 1, 192); }
  if (KT <= 32) { SVG_TRY(8, 4, 4, 128); else SVG_TRY(8, 4, 2, 192); }
  if (KT <= 64) { SVG_TRY(16, 4, 4, 128); else SVG_TRY(16, 4, 2, 128); }
  if (KT <= 96) {
    SVG_TRY(16, 6, 2, 128); else SVG_TRY(12, 8, 2, 168); else SVG_TRY(16, 6, 1, 128);
    else SVG_TRY(8, 12, 2, 256); else SVG_TRY(8, 12, 1, 256);
  }
  if (KT <= 128) { SVG_TRY(16, 8, 4, 128); else SVG_TRY(16, 8, 2, 128); }
  if (KT <= 192) { SVG_TRY(16, 12, 4, 128); else SVG_TRY(16, 12, 2, 128); else SVG_TRY(8, 24, 2, 256); }
#undef SVG_TRY
#undef SVG_FITS
  return launch_linear<P, 8, 0, 1>(a, f, stream);
}
