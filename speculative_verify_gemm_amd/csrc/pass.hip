// One pass of dependent W4A8 linears in one persistent launch (gfx950).
//
// Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
// (blog.dailydoseofds.com).  Section "Why batch-one decoding is memory-bound":
// a pass streams every weight once with about one multiply-add each, so the
// pass costs its bytes over the bandwidth -- provided the stream never stops.
// Section "How Uzu optimizes bytes and tokens per pass": activations are
// rotated (sign flips, then a +/-1 Hadamard per block) and quantized to int8
// on the fly; 4-bit asymmetric weights with one scale per group.  Section
// "Producing several tokens from one model pass": verification runs the same
// linears on 16-32 candidate rows.
//
// The problem this launch solves: the linears of a pass depend on each other
// (a step's input is ready only when the step before has finished), and on
// this chip a dependent kernel launch leaves HBM idle for several
// microseconds, 128-256 times per pass.  Weights depend on nothing, so here
// one launch runs the whole pass and keeps loading the NEXT steps' weights
// while a step waits for its input.
//
// One 1024-thread workgroup per compute unit, two roles:
//  * 12 stream waves: each keeps a ring of kRing weight chunks (1 KiB of
//    codes + their group parameters) in flight.  Its chunk sequence runs over
//    all steps: for each step, for each of the workgroup's 16-row tiles, the
//    wave's own range of K.  Loads run kRing chunks ahead of the computation,
//    across tile and step boundaries; computation reads the activation codes
//    from LDS and leaves fp32 partials per tile in LDS.
//  * 4 act waves: wait for a step's dependency, quantize its input rows into
//    LDS, sum the stream waves' partials of every tile in a fixed order
//    (deterministic), store y, and report the step done.  Their memory queue
//    holds no weight loads, so their own loads are not queued behind the
//    weight stream (loads return in issue order per wave).
// The two roles meet only at workgroup barriers, the same number on both
// sides: per step [dependency][quantization][one per tile][step end].
//
// Completion of a step: every workgroup counts itself in (one counter per
// group of workgroups, then one per step), after its y stores are performed
// device-wide (sc1 stores, then a wait for their acknowledgement).  "Step j
// counted complete" means every workgroup has finished steps 0..j, since each
// works through the steps in order.  A waiter polls with device-scope loads.
//
// Activations: M = 1: each workgroup's act waves rotate and quantize the row
// themselves (device-scope loads of X: it may be a previous step's output).
// M = 2..16: the rows are quantized once per XCC (the XCC each workgroup runs
// on is read from the hardware; workgroups of one XCC share its L2): a few
// workgroups of the XCC quantize one row each into that XCC's staging copy
// (plain stores: they stay in the XCC's L2), count themselves in, and every
// workgroup of the XCC copies the codes it needs into LDS with loads that
// bypass the compute unit's cache but are served by the XCC's L2.  Rows of
// M x K that do not fit LDS are cut along K in two halves; the workgroups of
// a pair each take one half of every tile, and the second to finish adds the
// two fp32 partials (half 0 first) and stores y.
//
// Every wait is bounded: a wait that gives up sets the workspace's first word
// and goes on, so the launch always ends.
#include <algorithm>

#include "../../include/svgemm.h"
#include "svg_act.h"
#include "svg_device.h"
#include "svg_internal.h"

namespace {

constexpr int kWaves = 16;
constexpr int kStreamWaves = 12;
constexpr int kThreads = kWaves * 64;
constexpr int kActThreads = (kWaves - kStreamWaves) * 64;
constexpr int kRing = 10;                 // weight chunks in flight per stream wave
constexpr int kPassMaxM = 16;
constexpr int kPassMaxK = 12288;
constexpr int kActLds = 110592;           // bytes of activation codes in LDS
constexpr int kSlots = 4;                 // tile partial slots (one per act wave)
constexpr int kStageRow = kPassMaxK;      // bytes per row of an XCC staging copy
constexpr int kXcc = 8;                   // counter groups (and XCC staging copies)
constexpr u32 kPollLimit = 1u << 20;      // device polls before a wait gives up (about a second)
constexpr u32 kMagic = 0x53564750u;       // plan image header

// The device image of one step (svg_pass_plan writes it on the host).
struct PassStep {
  const float* X;
  const int8_t* signs;
  int8_t* xq;
  float* x_scale;
  const uint8_t* wq;
  const uint16_t* ws;
  const void* wz;
  float* y;
  int32_t* dbg;
  int N, K, after, split;
  int KT, KH, cpw, KB;                    // chunks, chunks per half, chunks per stream wave, 512-k blocks
  int ntiles, kpad;                       // tiles; bytes per LDS activation row
  u32 part_off, tcnt_off;                 // split steps: partials and tile counters (workspace words)
  u32 wbytes, sbytes, zbytes, pad;
};
static_assert(sizeof(PassStep) == 136, "plan layout");

struct PassHdr {
  u32 magic;
  int nsteps, M, fmt, group, block;
  u32 ws_words, qbase, xbase, sbase;      // workspace regions (words)
  u32* trace;                             // optional: per (step, workgroup) phase times
  u32 pad[4];
};
static_assert(sizeof(PassHdr) == 64, "plan layout");

// Workspace (u32 words; counters 64 words = 256 bytes apart):
//   line 0: word 0 the give-up flag
//   lines 1..8: per-XCC tickets; line 9: start count
//   lines 10 + 9j .. 10 + 9j + 8: step j's group counters, then its total
//   lines qbase + 2j, + 2j + 1: step j's per-XCC quantization counts (16 words apart)
//   xbase: per-XCC staging rows (16 x kStageRow bytes each), sbase: scales
//   split steps: fp32 partials [tile][half][256] and tile counters
constexpr u32 kLine = 64;
SVG_DEV u32* ticket(u32* ws, int x) { return ws + kLine * (1 + x); }
SVG_DEV u32* start_count(u32* ws) { return ws + kLine * 9; }
SVG_DEV u32* group_count(u32* ws, int j, int g) { return ws + kLine * (10 + 9 * j + g); }
SVG_DEV u32* step_count(u32* ws, int j) { return ws + kLine * (10 + 9 * j + 8); }

SVG_DEV u32 ld_dev(const u32* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
SVG_DEV u32 add_dev(u32* p, u32 v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
SVG_DEV void st_dev(u32* p, u32 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
SVG_DEV void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier that waits only for this wave's LDS operations, not its
// global loads: the stream waves keep their weight loads in flight across it.
SVG_DEV void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Poll until *p >= target (device scope); false (and the flag set) if it
// gave up.  Once any wait has given up, every other wait stops early too.
SVG_DEV bool poll_ge(const u32* p, u32 target, u32* ws) {
  for (u32 it = 0; ld_dev(p) < target; ++it) {
    if ((it & 255u) == 255u && ld_dev(ws) != 0u) return false;
    if (it > kPollLimit) {
      st_dev(ws, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

// Stores through global-address-space pointers: a store through a generic
// pointer is a FLAT operation, which the compiler must assume may complete out
// of order with the weight loads -- every later wait on the ring would then
// drain it whole.
typedef __attribute__((address_space(1))) u32 global_u32;
typedef __attribute__((address_space(1))) int32_t global_i32;
SVG_DEV void gstore(u32* p, u32 v) { *(global_u32*)p = v; }
SVG_DEV void gstore(int32_t* p, int32_t v) { *(global_i32*)p = v; }
SVG_DEV void gstore(float* p, float v) { gstore(reinterpret_cast<u32*>(p), __float_as_uint(v)); }
typedef __attribute__((address_space(1))) float global_f32;
// An agent-scope store / load of a float through the global address space.
SVG_DEV void gstore_dev(float* p, float v) {
  __hip_atomic_store((global_f32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
SVG_DEV float gload_dev(const float* p) {
  return __hip_atomic_load((const global_f32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Phase timestamps (the 100 MHz real-time counter) for tracing a run: slot
// p of (step j, workgroup); a no-op unless the plan carries a trace buffer.
constexpr int kTracePhases = 8;
SVG_DEV void trace_at(u32* trace, int j, int p) {
  if (trace) gstore(trace + ((size_t)j * gridDim.x + blockIdx.x) * kTracePhases + p, (u32)__builtin_amdgcn_s_memrealtime());
}

// A value the same on every lane of the wave, said so to the compiler (its
// uniformity analysis cannot see through the spin loops on LDS counts in the
// stream waves' loop; state it thinks divergent would live in vector
// registers and cost a vector instruction per scalar one).
SVG_DEV int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
SVG_DEV u32 uni(u32 v) { return (u32)__builtin_amdgcn_readfirstlane((int)v); }
template <typename T>
SVG_DEV T* uni(T* p) {
  const uint64_t a = (uint64_t)p;
  return (T*)(((uint64_t)uni((u32)(a >> 32)) << 32) | uni((u32)a));
}

SVG_DEV u32 hw_xcc() { return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 7u; }

// Count this workgroup in as done with step j (one lane).  Returns true if it
// was the last workgroup of the final step (everything else has finished).
SVG_DEV bool arrive(u32* ws, int j, int nsteps) {
  const int G = gridDim.x, g = blockIdx.x & 7;
  const int gsize = (G - g + 7) / 8, ngroups = G < 8 ? G : 8;
  if (add_dev(group_count(ws, j, g), 1u) == (u32)gsize - 1)
    return add_dev(step_count(ws, j), 1u) == (u32)ngroups - 1 && j == nsteps - 1;
  return false;
}

// ---------------------------------------------------------------- geometry
// One step as one workgroup (and one stream wave) sees it.  Every workgroup
// walks the same number of tile slots in a step, ceil(tiles / workgroups per
// half of K); a slot past the last tile is walked without touching memory.
// So the walk is counters only, with no search for the next step a
// workgroup has work in (a loop between the weight loads and their use would
// hide from the compiler how many loads are still in flight).
struct Geo {
  int nts, t0, ts;       // tile slots: tiles t0, t0 + ts, ... (nts of them)
  int jrel0, len;        // the workgroup's chunks of K: [jrel0, jrel0 + len), the first held by the LDS rows
  int h;                 // split steps: the half of K this workgroup takes
  int tlim;              // tiles below tlim are real (0: none for this workgroup)
};

SVG_DEV Geo step_geo(const PassStep& S) {
  Geo g;
  const int G = gridDim.x, bid = blockIdx.x;
  if (S.split) {
    const int G2 = G / 2, p = bid >> 1;
    g.h = bid & 1;
    g.t0 = p;
    g.ts = G2;
    g.nts = (S.ntiles + G2 - 1) / G2;
    g.tlim = p < G2 ? S.ntiles : 0;  // an odd workgroup out has no pair
    g.jrel0 = g.h * S.KH;
    g.len = min(S.KH, S.KT - g.jrel0);
  } else {
    g.h = 0;
    g.t0 = bid;
    g.ts = G;
    g.nts = (S.ntiles + G - 1) / G;
    g.tlim = S.ntiles;
    g.jrel0 = 0;
    g.len = S.KT;
  }
  return g;
}

// Workgroup barriers of a step the workgroup has tiles in (the same on both
// roles).  M = 1: one when the stream waves have finished the previous step
// (the LDS rows are free), one when the new codes are in LDS.  M >= 2: only
// the second -- every step after the first waits for all earlier ones, which
// includes this workgroup's own stream waves (the per-XCC staging rows are
// shared by consecutive steps, so the rows of a step may only be quantized
// once every workgroup has read the previous step's).
SVG_DEV bool waits(const PassStep& S, int j, int M) { return j > 0 && (S.after || M > 1); }
SVG_DEV int rows_of(int rank, int nx, int M) { return rank < M ? (M - 1 - rank) / nx + 1 : 0; }

// ------------------------------------------------------------- stream side
// A stream wave's share of a step: in every tile slot, chunks [jb, jb + cw)
// of the tile (absolute chunk indices along K).  The workgroup's range of K
// (all of it, or one half) is cut among the 12 waves into runs that differ by
// at most one chunk, so no wave walks a chunk outside the matrix.  A wave left
// without chunks (K under 12 chunks) walks one chunk per tile slot through a
// resource of no bytes: zeros, no memory traffic.
SVG_DEV void wave_share(const Geo& g, int swave, int& jb, int& cw, bool& real) {
  const int q = g.len / kStreamWaves, rem = g.len % kStreamWaves;
  cw = q + (swave < rem ? 1 : 0);
  jb = g.jrel0 + swave * q + min(swave, rem);
  real = cw > 0;
  if (!real) {
    cw = 1;
    jb = g.jrel0;
  }
}

// The position of a stream wave's walk: step j (nsteps: past the end), tile
// slot ti of nts (tile t, stride ts; tiles from tlim on are not real), the
// wave's run of cw chunks from jb, and `left` chunks of the current slot still
// to go.  The walk is counters only (no search for the next step a workgroup
// has work in: a loop between the weight loads and their use would hide from
// the compiler how many loads are still in flight).
struct WalkPos {
  int j, ti, nts, t, ts, tlim;
  int jb, cw, left;
  bool real;
  // The current step's table entry, addressed through a uniform index so
  // that it is read with scalar loads (a vector load would be a memory
  // operation of unknown count in the stream waves' loop).
  SVG_DEV const PassStep* step(const PassStep* plan) const { return plan + __builtin_amdgcn_readfirstlane(j); }
  // Enter step `to`; false past the end, where the walk stays (`left` never
  // runs out again).  Every field is written on both paths, after the branch
  // (stores to different fields at the end of two branches get merged into
  // one store at a computed address, and then the whole stream context stays
  // in scratch memory).
  SVG_DEV bool enter(const PassStep* plan, int nsteps, int swave, int to) {
    const bool ok = to < nsteps;
    int nts_ = 0, t_ = 0, ts_ = 0, tlim_ = 0, jb_ = 0, cw_ = 0, left_ = 1 << 30;
    bool real_ = false;
    if (ok) {
      const Geo g = step_geo(plan[uni(to)]);
      nts_ = g.nts;
      t_ = g.t0;
      ts_ = g.ts;
      tlim_ = g.tlim;
      wave_share(g, swave, jb_, cw_, real_);
      left_ = cw_;
    }
    j = to;
    ti = 0;
    nts = nts_;
    t = t_;
    ts = ts_;
    tlim = tlim_;
    jb = jb_;
    cw = cw_;
    left = left_;
    real = real_;
    return ok;
  }
  // After the last chunk of a tile slot: the next slot (returns 0), the next
  // step (1) or the end (2).
  SVG_DEV int next_tile(const PassStep* plan, int nsteps, int swave) {
    if (++ti < nts) {
      t += ts;
      left = cw;
      return 0;
    }
    return enter(plan, nsteps, swave, j + 1) ? 1 : 2;
  }
  SVG_DEV bool tile_real() const { return real && t < tlim; }
  // Every field is the same on all lanes; say so after the walk moves.
  SVG_DEV void uniform() {
    j = uni(j);
    ti = uni(ti);
    nts = uni(nts);
    t = uni(t);
    ts = uni(ts);
    tlim = uni(tlim);
    jb = uni(jb);
    cw = uni(cw);
    left = uni(left);
    real = uni((int)real) != 0;
  }
};

// The issue side: the loads of one chunk (1 KiB of codes, this lane's 16
// bytes, plus the group parameters of its row), addressed by a per-lane part
// (voffset) and a scalar part stepped per chunk (soffset).  A tile slot that
// is not real, and everything past the end, loads at per-lane offsets beyond
// any buffer: zeros, no memory traffic.
template <int G, bool Z4>
struct Issuer {
  static constexpr int GPC = 128 / G, GPB = 4 * GPC;
  // The slot registers keep the width of their loads (a 16-bit scale or zero,
  // an 8-bit pair of 4-bit zeros): widened where the chunk is computed, not
  // where it is loaded, so that no slot's load has to land early.
  using SType = typename std::conditional<GPC == 2, u32, uint16_t>::type;
  using ZType = typename std::conditional<Z4, uint8_t, SType>::type;
  WalkPos p;
  int KT = 0, KB = 0;
  int jj = 0;                   // absolute chunk index of the next chunk
  u32 woff = 0, svi = 0;        // its codes byte offset and parameter index (scalar parts)
  u32 vw = kOOB, vs = kOOB, vz = kOOB;  // per-lane parts for this tile slot (beyond every buffer if not real)
  rsrc_t wr = make_rsrc(nullptr, 0u), sr = make_rsrc(nullptr, 0u), zr = make_rsrc(nullptr, 0u);

  // lane16: this lane's 16 bytes of a chunk; lanep: its row's part of the
  // parameter index (row r of the tile: r * GPB)
  SVG_DEV void start_tile(u32 lane16, u32 lanep) {
    jj = p.jb;
    woff = ((u32)p.t * (u32)KT + (u32)jj) * 1024u;
    svi = ((u32)p.t * (u32)KB + (u32)(jj >> 2)) * 16u * GPB + (u32)(jj & 3) * GPC;
    const bool on = p.tile_real();
    vw = on ? lane16 : kOOB;
    vs = on ? lanep * 2u : kOOB;
    vz = on ? (Z4 ? lanep >> 1 : lanep * 2u) : kOOB;
  }
  // After entering a step (or the end)
  SVG_DEV void take(const PassStep* plan, bool entered, u32 lane16, u32 lanep) {
    if (!entered) {
      vw = vs = vz = kOOB;
      return;
    }
    const PassStep* S = p.step(plan);
    KT = S->KT;
    KB = S->KB;
    wr = make_rsrc(S->wq, S->wbytes);
    sr = make_rsrc(S->ws, S->sbytes);
    zr = make_rsrc(S->wz, S->zbytes);
    start_tile(lane16, lanep);
  }
  SVG_DEV void issue(u32x4& wv, SType& s, ZType& z) const {
    wv = __builtin_amdgcn_raw_buffer_load_b128(wr, vw, woff, kNT);
    if constexpr (GPC == 2) {
      s = __builtin_amdgcn_raw_buffer_load_b32(sr, vs, svi * 2u, 0);
      if constexpr (Z4) z = __builtin_amdgcn_raw_buffer_load_b8(zr, vz, svi >> 1, 0);
      else z = __builtin_amdgcn_raw_buffer_load_b32(zr, vz, svi * 2u, 0);
    } else {
      s = __builtin_amdgcn_raw_buffer_load_b16(sr, vs, svi * 2u, 0);
      if constexpr (Z4) z = __builtin_amdgcn_raw_buffer_load_b8(zr, vz, svi >> 1, 0);
      else z = __builtin_amdgcn_raw_buffer_load_b16(zr, vz, svi * 2u, 0);
    }
  }
  SVG_DEV void uniform() {
    p.uniform();
    KT = uni(KT);
    KB = uni(KB);
    jj = uni(jj);
    woff = uni(woff);
    svi = uni(svi);
  }
  // Step to the next chunk: the next 1 KiB of codes; the parameters of the
  // next chunk of the 512-k block, or of the next block's first chunk.
  SVG_DEV void advance(const PassStep* plan, int nsteps, int swave, u32 lane16, u32 lanep) {
    woff += 1024u;
    svi += (jj & 3) == 3 ? (u32)(16 * GPB - 3 * GPC) : (u32)GPC;
    ++jj;
    if (--p.left == 0) {
      const int n = p.next_tile(plan, nsteps, swave);
      p.uniform();
      if (n == 0) start_tile(lane16, lanep);
      else take(plan, n == 1, lane16, lanep);
    }
  }
};

// The consume side: the chunk being computed and what its tile's hand-over
// needs.
template <int G, bool Z4>
struct Consumer {
  WalkPos p;
  int jj = 0;               // absolute chunk index of the current chunk
  int jrel0 = 0;            // first chunk of the LDS rows
  int N = 0, NG = 0, kpad = 0;
  int32_t* dbg = nullptr;
  int r = 0;

  // After entering a new tile slot (entered: of a new step)
  SVG_DEV void take(const PassStep* plan, bool entered) {
    jj = p.jb;
    if (!entered) return;
    const PassStep* S = p.step(plan);
    N = S->N;
    NG = S->K / G;
    kpad = S->kpad;
    dbg = S->dbg;
    jrel0 = S->split ? (blockIdx.x & 1) * S->KH : 0;
  }
  SVG_DEV void uniform() {
    p.uniform();
    jj = uni(jj);
    jrel0 = uni(jrel0);
    N = uni(N);
    NG = uni(NG);
    kpad = uni(kpad);
    dbg = uni(dbg);
  }
  SVG_DEV float scale(u32 s, int i) const { return half_bits_to_float((uint16_t)(i ? s >> 16 : s & 0xFFFF)); }
  // Zero of group i (0 or 1) of the chunk.  4-bit zeros of 128-wide groups:
  // the chunk's nibble is the odd one for odd chunks.
  SVG_DEV int zero(u32 z, int i) const {
    if constexpr (Z4) return (int)((z >> (G == 128 ? 4 * (jj & 1) : 4 * i)) & 0xF);
    else return (int)half_bits_to_float((uint16_t)(i ? z >> 16 : z & 0xFFFF));
  }
  // exact group sums are written for tests only, and only for real chunks
  SVG_DEV bool dbg_on() const { return dbg != nullptr && p.tile_real(); }
};

SVG_DEV void unpack8(u32 w, u32& lo, u32& hi) {
  lo = w & 0x0F0F0F0Fu;
  hi = (w >> 4) & 0x0F0F0F0Fu;
}
SVG_DEV v4i run_operand(u32 w0, u32 w1) {
  u32 a, b, c, d;
  unpack8(w0, a, b);
  unpack8(w1, c, d);
  return v4i{(int)a, (int)b, (int)c, (int)d};
}
SVG_DEV v4i neg_zero_operand(int z) {
  const u32 w = __builtin_amdgcn_perm(0u, (u32)(-z), 0x00000000u);
  return v4i{(int)w, (int)w, (int)w, (int)w};
}
SVG_DEV v4i mfma_i8(v4i a, v4i b, v4i c) { return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0); }
SVG_DEV v4i as_v4i(u32x4 a) { return v4i{(int)a[0], (int)a[1], (int)a[2], (int)a[3]}; }

// One chunk of the dot-product form (M = 1): lane (r, b) holds row r's two
// 16-k runs; the activation runs come from the LDS row.
template <int G, bool Z4>
SVG_DEV void compute_dot(const Consumer<G, Z4>& it, const u32x4& w, u32 s, u32 z, const int8_t* act, int b,
                         float& acc) {
  const int jrel = it.jj - it.jrel0;
  const u32x4 a1 = *reinterpret_cast<const u32x4*>(act + jrel * 128 + 16 * b);
  const u32x4 a2 = *reinterpret_cast<const u32x4*>(act + jrel * 128 + 64 + 16 * b);
  u32 wl[8];
  unpack8(w[0], wl[0], wl[1]);
  unpack8(w[1], wl[2], wl[3]);
  unpack8(w[2], wl[4], wl[5]);
  unpack8(w[3], wl[6], wl[7]);
  int p1 = 0, p2 = 0, q1 = 0, q2 = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    p1 = dot4(wl[k], a1[k], p1);
    p2 = dot4(wl[4 + k], a2[k], p2);
    q1 = dot4(a1[k], 0x01010101u, q1);
    q2 = dot4(a2[k], 0x01010101u, q2);
  }
  constexpr bool two = G == 64;  // g64: run 1 in group 2j, run 2 in group 2j + 1
  int S1 = p1 - it.zero(z, 0) * q1;
  int S2 = p2 - it.zero(z, two ? 1 : 0) * q2;
  acc = fmaf(it.scale(s, 0), (float)S1, acc);
  acc = fmaf(it.scale(s, two ? 1 : 0), (float)S2, acc);
  if (it.dbg_on()) {  // exact group sums for tests: add up the 4 lanes of each run
    if constexpr (!two) S1 += S2;
    S1 += lane_xor16(S1);
    S1 += lane_xor32(S1);
    S2 += lane_xor16(S2);
    S2 += lane_xor32(S2);
    const int n = it.p.t * 16 + it.r, jj = it.jj;
    if (b == 0 && n < it.N) {
      if (two) {
        if (2 * jj < it.NG) gstore(it.dbg + (size_t)n * it.NG + 2 * jj, S1);
        if (2 * jj + 1 < it.NG) gstore(it.dbg + (size_t)n * it.NG + 2 * jj + 1, S2);
      } else if (jj < it.NG) {
        gstore(it.dbg + (size_t)n * it.NG + jj, S1);
      }
    }
  }
}

// One chunk of the MFMA form (M = 2..16, rows past M are zero): A = 16
// tokens x 64 k from the LDS rows, B = the chunk's runs; the zero point is a
// second MFMA of the same A against -z in every byte.
template <int G, bool Z4>
SVG_DEV void compute_mfma(const Consumer<G, Z4>& it, const u32x4& w, u32 s, u32 z, const int8_t* act, int M, int b,
                          float (&acc)[4]) {
  const int jrel = it.jj - it.jrel0;
  const int r = it.r;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int8_t* row = act + (r < M ? r : 0) * it.kpad + jrel * 128 + 16 * b;
  const u32x4 x1 = *reinterpret_cast<const u32x4*>(row);
  const u32x4 x2 = *reinterpret_cast<const u32x4*>(row + 64);
  const v4i A1 = as_v4i(r < M ? x1 : zero), A2 = as_v4i(r < M ? x2 : zero);
  const v4i B1 = run_operand(w[0], w[1]), B2 = run_operand(w[2], w[3]);
  const v4i z4 = {0, 0, 0, 0};
  const v4i Z1 = neg_zero_operand(it.zero(z, 0));
  if constexpr (G == 64) {
    const v4i Z2 = neg_zero_operand(it.zero(z, 1));
    const v4i e1 = mfma_i8(A1, Z1, mfma_i8(A1, B1, z4));
    const v4i e2 = mfma_i8(A2, Z2, mfma_i8(A2, B2, z4));
    const float s1 = it.scale(s, 0), s2 = it.scale(s, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = fmaf(s1, (float)e1[i], acc[i]);
      acc[i] = fmaf(s2, (float)e2[i], acc[i]);
    }
    if (it.dbg_on()) {
      const int n = it.p.t * 16 + r, jj = it.jj;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * b + i;
        if (m < M && n < it.N) {
          if (2 * jj < it.NG) gstore(it.dbg + ((size_t)m * it.N + n) * it.NG + 2 * jj, e1[i]);
          if (2 * jj + 1 < it.NG) gstore(it.dbg + ((size_t)m * it.N + n) * it.NG + 2 * jj + 1, e2[i]);
        }
      }
    }
  } else {
    const v4i e = mfma_i8(A2, Z1, mfma_i8(A1, Z1, mfma_i8(A2, B2, mfma_i8(A1, B1, z4))));
    const float s1 = it.scale(s, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(s1, (float)e[i], acc[i]);
    if (it.dbg_on()) {
      const int n = it.p.t * 16 + r, jj = it.jj;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * b + i;
        if (m < M && n < it.N && jj < it.NG) gstore(it.dbg + ((size_t)m * it.N + n) * it.NG + jj, e[i]);
      }
    }
  }
}

// ------------------------------------------------------------------- LDS
struct PassLds {
  u32 act[kActLds / 4];                       // activation codes: M rows of kpad bytes
  float part[kSlots][kStreamWaves * 256];     // tile partials; slot s is summed by act wave s
  float xs[kPassMaxM];                        // row scales of the current step
  float red[kPassMaxM * 4];                   // act waves' maxima
  u32 ready[kSlots], consumed[kSlots];        // per slot: stream waves in, uses summed
  u32 act_done;                               // act waves' step-end count
  u32 act_sync;                               // act waves' own barrier count
  int rank, nx;                               // this workgroup's rank in its XCC, XCC size
};
// The workgroup's LDS, named at namespace scope so that every access is known
// to be an LDS access (through a generic pointer it would be a FLAT one, which
// the compiler must assume completes out of order with the weight loads).
__shared__ PassLds g_lds;

SVG_DEV u32 lds_ld(const u32* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
SVG_DEV void lds_add(u32* p, u32 v) { __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
SVG_DEV void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Spin until an LDS count reaches target; bounded like every other wait
// (true if it gave up).  The loop touches LDS only: a global access in a loop
// of the stream waves would hide from the compiler how many of their weight
// loads are still in flight, and every later wait would drain them all.
SVG_DEV bool lds_wait_ge(const u32* p, u32 target) {
  for (u32 it = 0; lds_ld(p) < target; ++it) {
    if (it > (1u << 23)) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// A barrier of the four act waves alone (the stream waves go on): an LDS
// count, each act wave adding one after its own LDS operations.
struct ActSync {
  u32* count;
  u32* ws;
  u32 phase;
  SVG_DEV void operator()(int lane) {
    lds_fence();
    if (lane == 0) lds_add(count, 1u);
    ++phase;
    if (lds_wait_ge(count, 4u * phase)) st_dev(ws, 1u);
    asm volatile("" ::: "memory");
  }
};

// ----------------------------------------------------------------- act side
// Rotate and quantize one row (K values) with the 256 act threads: CPT float4
// chunks per thread (chunk atid + 256 i).  Codes go to `put(word, value)`;
// returns nothing until the scale is known to every act wave, which needs one
// workgroup barrier (counted by the caller).  X is read with device-scope
// loads (it may have been written by an earlier step on another XCC).
template <int CPT, int B>
SVG_DEV float quant_row_regs(const float* X, int K, const int8_t* signs, float (&e)[CPT][4], int atid) {
  const rsrc_t xr = make_rsrc(X, (u32)K * 4u), sr = make_rsrc(signs, (u32)K);
  int sg[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const u32 c = (u32)atid + 256u * i;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, c * 16u, 0, kSC1);
    sg[i] = (int)bload4(sr, c * 4u);
    e[i][0] = __uint_as_float(v[0]); e[i][1] = __uint_as_float(v[1]);
    e[i][2] = __uint_as_float(v[2]); e[i][3] = __uint_as_float(v[3]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    apply_signs4(e[i][0], e[i][1], e[i][2], e[i][3], sg[i]);
    fwht_lane4<B>(e[i][0], e[i][1], e[i][2], e[i][3]);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(e[i][0]), fabsf(e[i][1])), fmaxf(fabsf(e[i][2]), fabsf(e[i][3]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  return amax;
}

template <int CPT, class Put>
SVG_DEV void codes_of_row(const float (&e)[CPT][4], int K, float amax, int atid, Put&& put) {
  const float sigma = amax / 127.0f;
  const float rinv = 1.0f / sigma;
  const bool fast = sigma >= 0x1p-125f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const u32 c = (u32)atid + 256u * i;
    if (c < (u32)K / 4u) {
      int q[4] = {0, 0, 0, 0};
      if (amax > 0.f) act_codes4(e[i], sigma, rinv, fast, q);
      put(c, pack4(q));
    }
  }
}

// Quantize the row (M = 1) into LDS; the workgroup barrier at the end says
// the codes are there.  Workgroup 0 also writes the step's xq / x_scale
// outputs.
template <int CPT, int B>
SVG_DEV void act_quant_m1(const PassStep& S, PassLds& L, int atid, int awave, ActSync& sync) {
  float e[CPT][4];
  const float wmax = quant_row_regs<CPT, B>(S.X, S.K, S.signs, e, atid);
  if ((atid & 63) == 0) L.red[awave] = wmax;
  sync(atid & 63);

  const float amax = fmaxf(fmaxf(L.red[0], L.red[1]), fmaxf(L.red[2], L.red[3]));
  const bool out = blockIdx.x == 0;
  u32* xq = reinterpret_cast<u32*>(S.xq);
  codes_of_row<CPT>(e, S.K, amax, atid, [&](u32 c, u32 v) {
    L.act[c] = v;
    if (out) gstore(xq + c, v);
  });
  for (int wd = S.K / 4 + atid; wd < S.kpad / 4; wd += kActThreads) L.act[wd] = 0u;  // zero past K
  if (atid == 0) {
    const float sc = (amax / 127.0f) * (1.0f / B);
    L.xs[0] = sc;
    if (out) gstore(S.x_scale, sc);
  }
  wg_barrier();
}

// Quantize row m (M >= 2) into this XCC's staging copy (act waves only); the
// first act thread counts the row in.  XCC 0's quantizers also write the
// step's xq (slab layout) / x_scale outputs.  The row goes through in groups
// of four float4 chunks per thread, its rotated values parked in the LDS rows
// (free until the codes are copied in) so that no more than one group is
// held in registers.
template <int B>
SVG_DEV void act_quant_row_stage(const PassStep& S, PassLds& L, int m, int M, u32* ws, const PassHdr& H, u32 xcc,
                                 int j, int atid, int awave, ActSync& sync) {
  float4* park = reinterpret_cast<float4*>(L.act);   // K / 4 float4 (<= 48 KiB)
  const int nchunk = S.K / 4, ngrp = (nchunk + 4 * 256 - 1) / (4 * 256);
  float wmax = 0.f;
  for (int gi = 0; gi < ngrp; ++gi) {
    float e[4][4];
    const int c0 = atid + 1024 * gi;  // chunks c0 + 256 i, i < 4
    const float mx = quant_row_regs<4, B>(S.X + (size_t)m * S.K + 4 * (size_t)(1024 * gi), S.K - 4 * 1024 * gi,
                                          S.signs + 4 * 1024 * gi, e, atid);
    wmax = fmaxf(wmax, mx);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + 256 * i < nchunk) park[c0 + 256 * i] = make_float4(e[i][0], e[i][1], e[i][2], e[i][3]);
  }
  if ((atid & 63) == 0) L.red[awave] = wmax;
  sync(atid & 63);
  const float amax = fmaxf(fmaxf(L.red[0], L.red[1]), fmaxf(L.red[2], L.red[3]));
  const float sigma = amax / 127.0f;
  const float rinv = 1.0f / sigma;
  const bool fast = sigma >= 0x1p-125f;
  u32* stage = ws + H.xbase + xcc * (kPassMaxM * kStageRow / 4) + m * (kStageRow / 4);
  const bool out = xcc == 0;
  u32* xq = reinterpret_cast<u32*>(S.xq);
  for (int c = atid; c < nchunk; c += 256) {
    const float4 f = park[c];
    const float u[4] = {f.x, f.y, f.z, f.w};
    int q[4] = {0, 0, 0, 0};
    if (amax > 0.f) act_codes4(u, sigma, rinv, fast, q);
    const u32 v = pack4(q);
    gstore(stage + c, v);
    if (out) gstore(xq + (((u32)c >> 3) * (u32)M + (u32)m) * 8u + ((u32)c & 7u), v);
  }
  if (atid == 0) {
    const float sc = sigma * (1.0f / B);
    gstore(reinterpret_cast<float*>(ws + H.sbase + xcc * kLine) + m, sc);
    if (out) gstore(S.x_scale + m, sc);
  }
  wait_stores();  // the codes and the scale are in the XCC's L2 before the count
  sync(atid & 63);
  if (atid == 0) add_dev(ws + kLine * (H.qbase + 2 * j) + 16 * xcc, 1u);
}

// Copy the M staged rows (this workgroup's range of K) into LDS.
SVG_DEV void act_copy_stage(const PassStep& S, const Geo& g, PassLds& L, int M, u32* ws, const PassHdr& H, u32 xcc,
                            int atid) {
  const u32* stage = ws + H.xbase + xcc * (kPassMaxM * kStageRow / 4);
  const rsrc_t sr = make_rsrc(stage, (u32)(kPassMaxM * kStageRow));
  const int wpr = S.kpad / 4;          // LDS words per row
  const int w0 = g.jrel0 * 32;         // first staged word of the range
  const int kw = S.K / 4;              // staged words per row
  for (int i = atid; i < M * (wpr / 4); i += kActThreads) {  // 16-byte pieces
    const int m = i / (wpr / 4), p = i % (wpr / 4);
    const int wd = w0 + 4 * p;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
        sr, wd < kw ? (u32)(m * (kStageRow / 4) + wd) * 4u : kOOB, 0, kSC1);
    *reinterpret_cast<u32x4*>(&L.act[m * wpr + 4 * p]) = v;
  }
  if (atid < M)
    L.xs[atid] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(ws + H.sbase + xcc * kLine, 64u), (u32)atid * 4u, 0, kSC1));
}

// Sum the stream waves' partials of tile t (fixed order) and store y; split
// steps exchange the halves through the workspace (one act wave does it all).
// `dot`: the partials are the dot-product form's (one per row and wave),
// else the matrix-core form's (16 tokens x 16 rows per wave).
SVG_DEV void finish_tile(const PassStep& S, const Geo& g, PassLds& L, int slot, int t, int M, bool dot, u32* ws,
                         int lane) {
  const float* part = L.part[slot];
  if (dot) {
    if (lane < 16) {
      float v = 0.f;
      for (int w = 0; w < kStreamWaves; ++w) v += part[w * 16 + lane];
      const int n = t * 16 + lane;
      if (n < S.N)
        gstore_dev(S.y + n, L.xs[0] * v);
    }
    return;
  }
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = lane + 64 * i;  // output (token o / 16, row o % 16)
    float a = 0.f;
    for (int w = 0; w < kStreamWaves; ++w) a += part[w * 256 + o];
    v[i] = a;
  }
  if (S.split) {
    float* mine = reinterpret_cast<float*>(ws + S.part_off) + ((size_t)t * 2 + g.h) * 256;
    const float* other = reinterpret_cast<const float*>(ws + S.part_off) + ((size_t)t * 2 + (g.h ^ 1)) * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      gstore_dev(mine + lane + 64 * i, v[i]);
    wait_stores();
    u32 old = 0;
    if (lane == 0) old = add_dev(ws + S.tcnt_off + t, 1u);
    old = __shfl(old, 0);
    if (old == 0) return;  // the other half finishes the tile
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = gload_dev(other + lane + 64 * i);
      v[i] = g.h == 0 ? v[i] + o : o + v[i];
    }
    if (lane == 0) st_dev(ws + S.tcnt_off + t, 0u);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = lane + 64 * i, m = o >> 4, n = t * 16 + (o & 15);
    if (m < M && n < S.N)
      gstore_dev(S.y + (size_t)m * S.N + n, L.xs[m] * v[i]);
  }
}

template <int B>
SVG_DEV void quant_m1_any(const PassStep& S, PassLds& L, int atid, int awave, ActSync& sync) {
  if (S.K <= 4096) act_quant_m1<4, B>(S, L, atid, awave, sync);
  else if (S.K <= 8192) act_quant_m1<8, B>(S, L, atid, awave, sync);
  else act_quant_m1<12, B>(S, L, atid, awave, sync);
}

// ------------------------------------------------------------- the ring
template <int G, bool Z4, bool MFMA>
struct StreamCtx {
  const PassStep* plan;
  u32* trace;
  int nsteps, M, wave, lane, b;
  u32 lane16, lanep;
  Issuer<G, Z4> iss;
  Consumer<G, Z4> con;
  u32x4 W[kRing];
  typename Issuer<G, Z4>::SType Sc[kRing];
  typename Issuer<G, Z4>::ZType Zr[kRing];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  u32 seq = 0;  // tile slots this workgroup has finished

  SVG_DEV void uniform() {
    nsteps = uni(nsteps);
    M = uni(M);
    wave = uni(wave);
    seq = uni(seq);
    iss.uniform();
    con.uniform();
  }
  // Wait until the codes of the step the consumer has just entered are in
  // LDS (M = 1: first until every stream wave is done with the previous row).
  SVG_DEV void wait_codes() {
    if constexpr (!MFMA) wg_barrier();
    wg_barrier();
    if (wave == 0 && lane == 0) trace_at(trace, con.p.j, 3);
  }
};

// Slot S of the ring, unrolled by recursion so that every register of the
// ring is named statically: compute the chunk in slot S, load the chunk
// kRing positions ahead into it, then move the consumer on (at the end of a
// tile slot: hand the partials over; on entering a step: wait for its codes,
// with this slot's load already on its way).
//
// The end of the sequence is tested in slot 0 only, and every slot issues its
// loads on every path (past the end they load zeros without touching
// memory), so on every path from a slot's loads back to that slot the same
// number of loads follow them: the compiler's wait before each chunk leaves
// the other kRing - 1 chunks in flight.  (An exit from the middle of the turn
// would join the loop's back edge with fewer loads behind the slot and force
// a wait for all of them.)  Past the end a slot computes on zeros from LDS
// offsets at most kRing chunks past the last row's end (inside the
// workgroup's LDS) and hands nothing over.
template <int G, bool Z4, bool MFMA, int S>
struct RingSlot {
  static SVG_DEV void load(StreamCtx<G, Z4, MFMA>& x) {
    x.iss.issue(x.W[S], x.Sc[S], x.Zr[S]);
    x.iss.advance(x.plan, x.nsteps, x.wave, x.lane16, x.lanep);
  }
  static SVG_DEV void prime(StreamCtx<G, Z4, MFMA>& x) {
    load(x);
    if constexpr (S + 1 < kRing) RingSlot<G, Z4, MFMA, S + 1>::prime(x);
  }
  // One turn; false once the sequence has ended.
  static SVG_DEV bool run(StreamCtx<G, Z4, MFMA>& x) {
    Consumer<G, Z4>& it = x.con;
    if constexpr (S == 0) {
      x.uniform();
      if (it.p.j >= x.nsteps) return false;
    }
    const bool live = S == 0 || it.p.j < x.nsteps;
    const int8_t* act = reinterpret_cast<const int8_t*>(g_lds.act);
    if constexpr (MFMA) compute_mfma<G, Z4>(it, x.W[S], x.Sc[S], x.Zr[S], act, x.M, x.b, x.acc);
    else compute_dot<G, Z4>(it, x.W[S], x.Sc[S], x.Zr[S], act, x.b, x.acc[0]);
    load(x);
    if (live) {
      ++it.jj;
      if (--it.p.left == 0 && hand_over(x)) x.wait_codes();
    }
    if constexpr (S + 1 < kRing) return RingSlot<G, Z4, MFMA, S + 1>::run(x);
    else return true;
  }
  // The wave's last chunk of a tile slot is in: its partials go to the
  // slot's LDS entry (once the act wave has summed the entry's previous use).
  // Returns true when the walk entered a new step.
  static SVG_DEV bool hand_over(StreamCtx<G, Z4, MFMA>& x) {
    Consumer<G, Z4>& it = x.con;
    const u32 slot = x.seq % kSlots, use = x.seq / kSlots;
    lds_wait_ge(&g_lds.consumed[slot], use);  // a give-up shows on the act side
    float* part = g_lds.part[slot];
    if constexpr (MFMA) {
#pragma unroll
      for (int i = 0; i < 4; ++i) part[x.wave * 256 + (4 * x.b + i) * 16 + it.r] = x.acc[i];
    } else {
      float v = x.acc[0];
      v += lane_xorf<16>(v);
      v += __int_as_float(lane_xor32(__float_as_int(v)));
      if (x.b == 0) part[x.wave * 16 + it.r] = v;
    }
    lds_fence();
    if (x.lane == 0) lds_add(&g_lds.ready[slot], 1u);
    x.acc[0] = x.acc[1] = x.acc[2] = x.acc[3] = 0.f;
    ++x.seq;
    if (x.wave == 0 && x.lane == 0 && it.p.ti == it.p.nts - 1) trace_at(x.trace, it.p.j, 7);
    const int n = it.p.next_tile(x.plan, x.nsteps, x.wave);
    it.p.uniform();
    it.take(x.plan, n == 1);
    return n == 1;
  }
};

// ------------------------------------------------------------------ kernel
template <int G, bool Z4, bool MFMA>
__global__ __launch_bounds__(kThreads, 1) void k_pass(const PassHdr* __restrict__ hdr_p, u32* ws) {
  PassLds& L = g_lds;
  const PassHdr H = *hdr_p;
  const PassStep* plan = reinterpret_cast<const PassStep*>(hdr_p + 1);
  const int nsteps = H.nsteps, M = H.M;
  // the wave index is uniform over the wave: say so, so that everything the
  // walks derive from it (and the step table loads) stays scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const u32 xcc = hw_xcc();
  if (threadIdx.x < kSlots) {
    L.ready[threadIdx.x] = 0u;
    L.consumed[threadIdx.x] = 0u;
  }
  if (threadIdx.x == 0) {
    L.act_done = 0u;
    L.act_sync = 0u;
  }
  wg_barrier();

  if (wave < kStreamWaves) {
    // ------------------------------------------------------ stream waves
    StreamCtx<G, Z4, MFMA> x;
    x.plan = plan;
    x.trace = H.trace;
    x.nsteps = nsteps;
    x.M = M;
    x.wave = wave;
    x.lane = lane;
    x.b = lane >> 4;
    x.lane16 = (u32)lane * 16u;
    x.lanep = (u32)(lane & 15) * (u32)Issuer<G, Z4>::GPB;
    x.iss.take(plan, x.iss.p.enter(plan, nsteps, wave, 0), x.lane16, x.lanep);
    x.con.r = lane & 15;
    x.con.p = x.iss.p;
    x.con.take(plan, true);                 // step 0 (the pass has at least one step)
    RingSlot<G, Z4, MFMA, 0>::prime(x);   // the issue side runs kRing chunks ahead
    if (M > 1) wg_barrier();               // start: the XCC ranks are known
    x.wait_codes();
    while (RingSlot<G, Z4, MFMA, 0>::run(x)) {
    }
  } else {
    // --------------------------------------------------------- act waves
    const int atid = threadIdx.x - kStreamWaves * 64, awave = wave - kStreamWaves;
    if (M > 1) {
      if (atid == 0) {
        const u32 rank = add_dev(ticket(ws, xcc), 1u);
        add_dev(start_count(ws), 1u);
        poll_ge(start_count(ws), gridDim.x, ws);
        L.rank = (int)rank;
        L.nx = (int)ld_dev(ticket(ws, xcc));
      }
      wg_barrier();
    }
    const int rank = M > 1 ? L.rank : 0, nxc = M > 1 ? L.nx : 1;
    bool last = false;
    u32 seq = 0, steps_done = 0;
    ActSync sync{&L.act_sync, ws, 0u};
    for (int j = 0; j < nsteps; ++j) {
      const PassStep& S = plan[j];
      const Geo g = step_geo(S);
      if constexpr (!MFMA) {  // M = 1: each workgroup quantizes the row it needs
        if (atid == 0) trace_at(H.trace, j, 0);
        wg_barrier();  // the stream waves are done with the previous step's LDS row
        if (waits(S, j, M)) {  // every earlier step counted complete
          if (atid == 0) poll_ge(step_count(ws, j - 1), (u32)(gridDim.x < 8 ? gridDim.x : 8), ws);
          sync(lane);
        }
        if (atid == 0) trace_at(H.trace, j, 1);
        if (H.block == 64) quant_m1_any<64>(S, L, atid, awave, sync);
        else quant_m1_any<32>(S, L, atid, awave, sync);
        if (atid == 0) {
          trace_at(H.trace, j, 2);
          trace_at(H.trace, j, 4);
        }
      } else if constexpr (MFMA) {  // M >= 2: rows quantized once per XCC, by workgroups with or without tiles
        if (atid == 0) trace_at(H.trace, j, 0);
        if (waits(S, j, M)) {
          if (atid == 0) poll_ge(step_count(ws, j - 1), (u32)(gridDim.x < 8 ? gridDim.x : 8), ws);
          sync(lane);
        }
        if (atid == 0) trace_at(H.trace, j, 1);
        for (int m = rank; m < M; m += nxc) {
          if (H.block == 64) act_quant_row_stage<64>(S, L, m, M, ws, H, xcc, j, atid, awave, sync);
          else act_quant_row_stage<32>(S, L, m, M, ws, H, xcc, j, atid, awave, sync);
        }
        if (atid == 0) trace_at(H.trace, j, 2);
        if ((atid & 63) == 0) poll_ge(ws + kLine * (H.qbase + 2 * j) + 16 * xcc, (u32)M, ws);
        act_copy_stage(S, g, L, M, ws, H, xcc, atid);
        wg_barrier();  // the codes are in LDS
        if (atid == 0) trace_at(H.trace, j, 4);
      }
      // tile slots: act wave s sums the partials of LDS slot s once all stream
      // waves are in (and stores y for a real tile)
      for (int ti = 0; ti < g.nts; ++ti, ++seq) {
        const u32 slot = seq % kSlots, use = seq / kSlots;
        if (awave != (int)slot) continue;
        if (lds_wait_ge(&L.ready[slot], kStreamWaves * (use + 1))) st_dev(ws, 1u);
        asm volatile("" ::: "memory");
        const int t = g.t0 + ti * g.ts;
        if (t < g.tlim) finish_tile(S, g, L, slot, t, M, !MFMA, ws, lane);
        lds_fence();
        if (lane == 0) __hip_atomic_store(&L.consumed[slot], use + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      // y performed device-wide (every act wave), then the step is counted
      if (atid == 0) trace_at(H.trace, j, 5);
      wait_stores();
      if (lane == 0) lds_add(&L.act_done, 1u);
      ++steps_done;
      if (atid == 0) {
        if (lds_wait_ge(&L.act_done, 4u * steps_done)) st_dev(ws, 1u);
        last = arrive(ws, j, nsteps);
        trace_at(H.trace, j, 6);
      }
    }
    // The last workgroup of the final step resets every counter for the next
    // run (all others have finished all their waits by then).
    if (awave == 0) {
      last = __shfl(last ? 1 : 0, 0) != 0;
      if (last) {
        for (u32 i = 1 + lane; i < 10 + 9u * nsteps; i += 64) st_dev(ws + kLine * i, 0u);
        for (int i = lane; i < nsteps * kXcc; i += 64) st_dev(ws + kLine * (H.qbase + 2 * (i / kXcc)) + 16 * (i % kXcc), 0u);
      }
    }
  }
}

template <int G, bool Z4>
hipError_t launch_g(const void* plan, int M, u32* ws, hipStream_t stream) {
  const int cus = svg_cu_count();
  const PassHdr* h = static_cast<const PassHdr*>(plan);
  if (M > 1) {
    constexpr auto k = k_pass<G, Z4, true>;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, kThreads, 0) != hipSuccess || occ < 1)
      return hipErrorLaunchOutOfResources;
    hipLaunchKernelGGL(k, dim3(cus), dim3(kThreads), 0, stream, h, ws);
  } else {
    constexpr auto k = k_pass<G, Z4, false>;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k, kThreads, 0) != hipSuccess || occ < 1)
      return hipErrorLaunchOutOfResources;
    hipLaunchKernelGGL(k, dim3(cus), dim3(kThreads), 0, stream, h, ws);
  }
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------- host
static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Workspace words and the split partial offsets for a pass (host).  Returns
// the total words; fills the per-step offsets when `img` is given.
static u32 pass_layout(const svg_pass_step* steps, int nsteps, int M, int group, int cus, PassHdr* hdr,
                       PassStep* img) {
  uint64_t words = kLine * (10 + 9ull * nsteps);
  hdr->qbase = (u32)ceil_div(words, kLine);
  words = kLine * ((uint64_t)hdr->qbase + 2ull * nsteps);
  hdr->xbase = (u32)words;
  if (M > 1) words += (uint64_t)kXcc * kPassMaxM * kStageRow / 4;
  hdr->sbase = (u32)words;
  if (M > 1) words += (uint64_t)kXcc * kLine;
  for (int j = 0; j < nsteps; ++j) {
    const int K = steps[j].K, N = steps[j].N;
    const int KT = (K + 127) / 128, ntiles = (N + 15) / 16;
    const int cpw_full = (int)ceil_div(KT, kStreamWaves);
    const int split = (M > 1 && (uint64_t)M * kStreamWaves * cpw_full * 128 > kActLds) ? 1 : 0;
    const int KH = split ? (KT + 1) / 2 : KT;
    const int cpw = (int)ceil_div(KH, kStreamWaves);
    if (img) {
      PassStep& p = img[j];
      p.split = split;
      p.KT = KT;
      p.KH = KH;
      p.cpw = cpw;
      p.KB = (K + kMetaK - 1) / kMetaK;
      p.ntiles = ntiles;
      p.kpad = kStreamWaves * cpw * 128;
      p.part_off = p.tcnt_off = 0;
    }
    if (split) {
      words = ceil_div(words, kLine) * kLine;
      if (img) img[j].part_off = (u32)words;
      words += (uint64_t)ntiles * 2 * 256;
      if (img) img[j].tcnt_off = (u32)words;
      words += ntiles;
    }
  }
  (void)group;
  (void)cus;
  return (u32)ceil_div(words, kLine) * kLine;
}

const char* svg_pass_check(const svg_pass_step* steps, int nsteps, int M, int fmt, int group, int block,
                           uint64_t* plan_bytes, uint64_t* ws_bytes, int* code) {
  *code = SVG_EINVAL;
  if (!steps) return "null steps";
  if (nsteps < 1) { *code = SVG_EUNSUPPORTED; return "nsteps < 1"; }
  if (nsteps > 100000) { *code = SVG_EUNSUPPORTED; return "more than 100000 steps"; }
  if (M < 1) return "M < 1";
  *code = SVG_EUNSUPPORTED;
  if (M > kPassMaxM) return "M > 16";
  if (fmt != SVG_W4_ASYM_Z4 && fmt != SVG_W4_ASYM_Z16) return "fmt must be a W4 format";
  if (group != 64 && group != 128) return "group must be 64 or 128";
  if (block != 32 && block != 64) return "block must be 32 or 64";
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  for (int j = 0; j < nsteps; ++j) {
    const svg_pass_step& s = steps[j];
    *code = SVG_EINVAL;
    if (!s.X || !s.signs || !s.xq || !s.x_scale || !s.wq || !s.w_scale || !s.w_zero || !s.y)
      return "a step has a null required pointer";
    if (s.N < 1 || s.K < 1) return "a step has N < 1 or K < 1";
    if (s.after != 0 && s.after != 1) return "a step's `after` is not 0 or 1";
    *code = SVG_EUNSUPPORTED;
    if (s.K % 32 || s.K % group || s.K % block) return "a step's K is not a multiple of 32, group and block";
    if (s.K > kPassMaxK) return "a step's K is above 12288";
    size_t wb, sb, zb;
    svg_w4_storage(s.N, s.K, group, fmt == SVG_W4_ASYM_Z4, &wb, &sb, &zb);
    if (wb >= (1ull << 32) || sb >= (1ull << 32) || zb >= (1ull << 32))
      return "a step's weight storage reaches 4 GiB";
    *code = SVG_EALIGN;
    if (!al(s.X, 16) || !al(s.xq, 16) || !al(s.wq, 16)) return "a step's X, xq or wq is not 16-byte aligned";
    if (!al(s.signs, 4) || !al(s.x_scale, 4) || !al(s.w_scale, 4) || !al(s.y, 4) ||
        (fmt == SVG_W4_ASYM_Z16 && !al(s.w_zero, 4)) || (s.partials_debug && !al(s.partials_debug, 4)))
      return "a step's signs, x_scale, w_scale, w_zero, y or partials pointer is misaligned";
  }
  PassHdr h{};
  const uint64_t words = pass_layout(steps, nsteps, M, group, svg_cu_count(), &h, nullptr);
  *plan_bytes = sizeof(PassHdr) + (uint64_t)nsteps * sizeof(PassStep);
  *ws_bytes = words * 4;
  *code = SVG_OK;
  return nullptr;
}

void svg_pass_write(const svg_pass_step* steps, int nsteps, int M, int fmt, int group, int block, void* plan_host) {
  PassHdr* h = static_cast<PassHdr*>(plan_host);
  PassStep* img = reinterpret_cast<PassStep*>(h + 1);
  *h = PassHdr{};
  h->magic = kMagic;
  h->nsteps = nsteps;
  h->M = M;
  h->fmt = fmt;
  h->group = group;
  h->block = block;
  for (int j = 0; j < nsteps; ++j) {
    const svg_pass_step& s = steps[j];
    PassStep& p = img[j];
    p = PassStep{};
    p.X = s.X; p.signs = s.signs; p.xq = s.xq; p.x_scale = s.x_scale;
    p.wq = s.wq; p.ws = s.w_scale; p.wz = s.w_zero; p.y = s.y; p.dbg = s.partials_debug;
    p.N = s.N; p.K = s.K; p.after = s.after;
    size_t wb, sb, zb;
    svg_w4_storage(s.N, s.K, group, fmt == SVG_W4_ASYM_Z4, &wb, &sb, &zb);
    p.wbytes = (u32)wb; p.sbytes = (u32)sb; p.zbytes = (u32)zb;
  }
  h->ws_words = pass_layout(steps, nsteps, M, group, svg_cu_count(), h, img);
}

hipError_t svg_launch_pass(const void* plan, int M, int fmt, int group, void* ws, hipStream_t stream) {
  u32* w = static_cast<u32*>(ws);
  const bool z4 = fmt == SVG_W4_ASYM_Z4;
  if (group == 64) return z4 ? launch_g<64, true>(plan, M, w, stream) : launch_g<64, false>(plan, M, w, stream);
  return z4 ? launch_g<128, true>(plan, M, w, stream) : launch_g<128, false>(plan, M, w, stream);
}
