/*
 * svgemm.h -- C ABI of the MI355X (gfx950) RHT + W4A8 / W8A8 quantized linear.
 *
 * Sources.  [KT] is the page "Karpathy's Trick for Faster Local LLMs Finally
 * Has Proper Tooling" (blog.dailydoseofds.com).  The three operations follow
 * its section "How Uzu optimizes bytes and tokens per pass": weights are
 * rotated by a block-diagonal random Hadamard transform (random sign flips,
 * then a +/-1 Hadamard on each block of 32) and quantized as 4-bit asymmetric
 * ("Medium") or 8-bit symmetric ("Large") integers; activations are rotated
 * the same way and quantized to int8 on the fly; the matmul is integer x
 * integer.  Its section "Producing several tokens from one model pass" sets the
 * verify sizes (16 to 32 candidate rows instead of 1).
 *
 * Conventions shared by every entry point:
 *  - Every pointer is a DEVICE pointer; the caller owns all memory.  Nothing
 *    is allocated, freed or synchronised inside a call.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream).  They may be captured in a HIP graph: no call records
 *    a memset or a host round trip.
 *  - Arguments are validated on the host before anything is enqueued; a failed
 *    check returns its status, sets svg_last_error(), and leaves every output
 *    untouched.  M == 0 or N == 0 is a valid empty call (nothing enqueued).
 *  - Outputs are overwritten, never accumulated.  Inputs and outputs must not
 *    overlap.
 *  - Numerics: the transform and every quantizer use IEEE fp32 add, subtract
 *    and divide with round-to-nearest-even and no fused multiply-add, so the
 *    integer codes are reproducible bit for bit; NaN/Inf inputs are outside
 *    the contract.
 *
 * The rotation is unnormalised (entries +/-1); the overall scale of the
 * transform on both operands, 1/sqrt(B) twice = 1/B for a transform block of
 * B values (2^-5 for the pages' B = 32), is folded exactly into x_scale.  One
 * Hadamard ordering is used throughout: Sylvester natural order,
 * H[i][j] = (-1)^popcount(i & j).  B = 64 is a variant sized to the 64-lane
 * wave (the pages size the block to their 32-wide SIMD group): the butterfly
 * has one more stage (h = 32).  Weights and the activations they meet must
 * use the same B.
 */
#ifndef SVGEMM_H
#define SVGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int svg_status;

enum {
    SVG_OK = 0,
    SVG_EINVAL = 1,        /* null required pointer, negative size, K <= 0      */
    SVG_EUNSUPPORTED = 2,  /* K > 2^24, a weight array of 4 GiB or more,
                              block not 32 or 64, K % 32, K % block, K % group, group not in
                              {32, 64, 128}, M > 32, unknown fmt, W8 K > 131072 */
    SVG_EALIGN = 3,        /* a pointer below its required alignment          */
    SVG_EHIP = 4           /* a HIP launch or runtime error (text in
                              svg_last_error())                               */
};

enum {
    SVG_W4_ASYM_Z4 = 0,   /* 4-bit asymmetric codes, fp16 scale, 4-bit zero      */
    SVG_W4_ASYM_Z16 = 1,  /* 4-bit asymmetric codes, fp16 scale, fp16 zero       */
    SVG_W8_SYM = 2        /* 8-bit symmetric codes, one fp16 scale per row       */
};

/*
 * Weight storage ("tiled"; the pages give no layout -- this one lets a wave read
 * each 16-row tile of a matrix as contiguous KiB in the lane order of the
 * int8 MFMA, v_mfma_i32_16x16x64_i8).
 *
 * W4 codes (wq): rows padded to Np = ceil(N/16)*16 and K to Kp = ceil(K/128)*128
 *   with code 0.  Tile (i, j) -- rows 16i..16i+15, k 128j..128j+127 -- is the
 *   1024 bytes at (i*Kp/128 + j)*1024.  Its 16-byte piece p = 16b + r
 *   (b = 0..3, r = 0..15) belongs to row 16i + r: bytes 0..7 hold
 *   k in [128j+16b, +16), bytes 8..15 hold k in [128j+64+16b, +16).  A 4-byte
 *   word covering k0..k0+7 holds code k0+t in the low nibble and code k0+t+4 in
 *   the high nibble of byte t.  Size Np*Kp/2 bytes.
 * W4 scales (fp16) and fp16 zeros: one value per (row, group); rows padded
 *   to 16 and K to a multiple of 512 with 0.  The 512/group values of
 *   (16-row tile i, 512-k block jb, row r) are contiguous, blocks ordered by
 *   (i, jb, r): value (n, g) sits at ((i*KB + jb)*16 + r)*(512/group) + c with
 *   i = n/16, r = n%16, jb = g/(512/group), c = g%(512/group), KB = ceil(K/512).
 *   Size Np*KB*(512/group) values.
 * W4 4-bit zeros: the same order, two per byte (even index in the low nibble).
 * W8 codes: rows padded to 16 and K to Kp8 = ceil(K/64)*64 with 0; tile (i, j)
 *   -- 16 rows x 64 k -- is 1024 bytes at (i*Kp8/64 + j)*1024; piece 16b + r
 *   holds row 16i + r, k in [64j+16b, +16) in natural order.  W8 scales: fp16
 *   [N] in row order.
 *
 * svg_weight_sizes gives the byte sizes a caller must allocate (host-only;
 * touches no device).  SVG_EINVAL / SVG_EUNSUPPORTED as for
 * rht_rotate_weights; zero_bytes is 0 for W8.
 */
svg_status svg_weight_sizes(int N, int K, int fmt, int group, uint64_t* wq_bytes,
                            uint64_t* scale_bytes, uint64_t* zero_bytes);

/*
 * rht_rotate_weights -- offline: rotate and quantize the rows of W.
 * [KT "How Uzu optimizes bytes and tokens per pass": the transform is applied
 *  before quantization; Medium = 4-bit asymmetric, Large = 8-bit symmetric.]
 *
 *  W        fp32 [N][K] row-major; row n is output channel n, contiguous in K.
 *           16-byte aligned.
 *  signs    int8 [K], each +1 or -1; the same vector must be given to
 *           act_rht_quant_i8 for the activations this matrix consumes.
 *           4-byte aligned.
 *  block    transform block, 32 (the pages') or 64; K must be a multiple of it.
 *  fmt      SVG_W4_ASYM_Z4, SVG_W4_ASYM_Z16 or SVG_W8_SYM.
 *  group    W4: quantization group along K, 32, 64 or 128 (independent of the
 *           transform block).  Ignored for W8.
 *  wq, w_scale, w_zero  outputs in the tiled storage above, sized by
 *           svg_weight_sizes; wq 16-byte aligned, w_scale and fp16 w_zero
 *           4-byte aligned; w_zero unused (may be NULL) for W8.  Padding is
 *           written as zeros.
 *  w_rot_debug  nullable fp32 [N][K]: receives the rotated rows u (tests).
 *
 *  Per row, u = H_B . diag(signs) . W[n] blockwise (butterfly stages
 *  h = 1, 2, 4, ..., B/2 in that order).  W4 per group: lo = min(0, min u),
 *  hi = max(0, max u), s = fp16(rne((hi - lo) / 15)) (1.0 if zero),
 *  z = clamp(rint(-lo / s), 0, 15) (a 4-bit unsigned value; -lo / s passes
 *  15 only when s is an fp16 subnormal), q = clamp(rint(u / s) + z, 0, 15).  W8 per row:
 *  s = fp16(rne(max|u| / 127)) (1.0 if zero), q = clamp(rint(u / s), -127, 127).
 *  Matrices whose rows are stacked along N (e.g. the q, k and v projections)
 *  may be rotated one at a time into consecutive 16-row tiles of one buffer
 *  when each has a multiple of 16 rows.
 */
svg_status rht_rotate_weights(const float* W, int N, int K, const int8_t* signs,
                              int block, int fmt, int group, void* wq,
                              uint16_t* w_scale, void* w_zero, float* w_rot_debug,
                              void* stream);

/*
 * act_rht_quant_i8 -- online: rotate the activation rows and quantize each to
 * int8 with one scale per row (token).
 * [KT "How Uzu optimizes bytes and tokens per pass": activations are quantized
 *  to 8 bits on the fly.]
 *
 *  X        fp32 [M][K] row-major, 16-byte aligned.  M <= 32.
 *  signs    int8 [K] (+/-1), 4-byte aligned; the weights' sign vector.
 *  block    32 or 64, as for the weights this row meets; K % block == 0.
 *  xq       M*K int8 codes in [-127, 127], 16-byte aligned, in 32-k slabs:
 *           the code of (row m, k) is byte ((k / 32) * M + m) * 32 + k % 32,
 *           i.e. slab s = k / 32 holds the 32 codes of row 0, then row 1, ...
 *           (for M = 1 this is the row itself).  The linears read 16 rows of
 *           a 64-k run as two contiguous 512-byte pieces this way.
 *  x_scale  fp32 [M]: (max_k |u| / 127) / block (0 for an all-zero row);
 *           4-byte aligned.
 *
 *  u = H_B . diag(signs) . X[m] blockwise; sigma = max|u| / 127;
 *  q = clamp(rint(u / sigma), -127, 127) (0 if the row is zero).
 */
svg_status act_rht_quant_i8(const float* X, int M, int K, const int8_t* signs,
                            int block, int8_t* xq, float* x_scale, void* stream);

/*
 * w4a8_linear -- y = x . W^T for int8 activations and W4 asymmetric weights.
 * [KT "How Uzu optimizes bytes and tokens per pass": both operands are
 *  integers and the product runs on the int8 matrix path; "Why batch-one
 *  decoding is memory-bound": each pass streams every weight once.]
 *
 *  xq, x_scale   from act_rht_quant_i8 (slab layout, xq 16-byte aligned),
 *                M in 1..32.
 *  wq, w_scale, w_zero, fmt (SVG_W4_ASYM_Z4 or _Z16), group: the tiled
 *                storage from rht_rotate_weights with the same signs, N rows,
 *                K columns (wq 16-byte, w_scale and fp16 w_zero 4-byte aligned).
 *  y             fp32 [M][N], 4-byte aligned.
 *  partials_debug  nullable int32 [M][N][K/group]: receives
 *                S_g[m][n] = sum_{k in g} xq[m][k] * (q[n][k] - z[n][g]),
 *                exact (tests).
 *
 *  y[m][n] = x_scale[m] * sum_g s[n][g] * S_g[m][n]  (fp32 accumulation; the
 *  integer partial sums are exact, the float sum is order-dependent only).
 */
svg_status w4a8_linear(const int8_t* xq, const float* x_scale, int M, int K,
                       const uint8_t* wq, const uint16_t* w_scale, const void* w_zero,
                       int fmt, int group, int N, float* y, int32_t* partials_debug,
                       void* stream);

/*
 * w8a8_linear -- y = x . W^T for int8 activations and W8 symmetric weights.
 * [KT "How Uzu optimizes bytes and tokens per pass": Large checkpoints are
 *  8-bit symmetric; both operands are integers.]
 *
 *  xq, x_scale   from act_rht_quant_i8 (slab layout, xq 16-byte aligned),
 *                M in 1..32.
 *  wq            tiled int8 codes from rht_rotate_weights (SVG_W8_SYM),
 *                16-byte aligned; w_scale fp16 bits [N].  K <= 131072 (so
 *                that |S| <= 127^2 K fits int32).
 *  y             fp32 [M][N].
 *  partials_debug  nullable int32 [M][N]: S[m][n] = sum_k xq[m][k] * q[n][k].
 *
 *  y[m][n] = x_scale[m] * s[n] * S[m][n].
 */
svg_status w8a8_linear(const int8_t* xq, const float* x_scale, int M, int K,
                       const int8_t* wq, const uint16_t* w_scale, int N, float* y,
                       int32_t* partials_debug, void* stream);

/*
 * act_quant_w4a8_linear, act_quant_w8a8_linear -- act_rht_quant_i8 followed by
 * w4a8_linear / w8a8_linear, taking the fp32 activation rows directly.
 * [KT "How Uzu optimizes bytes and tokens per pass": activations quantized on
 *  the fly; "Why batch-one decoding is memory-bound": a decode pass is the
 *  weight stream, so the activation step should not cost a launch of its own.]
 *
 *  X, signs, block   as for act_rht_quant_i8.
 *  xq, x_scale       OUTPUTS here (as from act_rht_quant_i8), then read by the
 *                    contraction; the results are bit-identical to the two
 *                    separate calls.
 *  wq ... partials_debug   as for w4a8_linear / w8a8_linear.
 *
 *  For M = 1 (M <= 2 with 32-wide groups) and K <= 12288 this is ONE launch:
 *  every workgroup quantizes the row itself while its first weights are in
 *  flight.  Otherwise it enqueues the two launches.  Errors as for the two separate calls; N == 0 runs the
 *  quantization alone.
 */
svg_status act_quant_w4a8_linear(const float* X, int M, int K, const int8_t* signs, int block,
                                 int8_t* xq, float* x_scale, const uint8_t* wq,
                                 const uint16_t* w_scale, const void* w_zero, int fmt, int group,
                                 int N, float* y, int32_t* partials_debug, void* stream);
svg_status act_quant_w8a8_linear(const float* X, int M, int K, const int8_t* signs, int block,
                                 int8_t* xq, float* x_scale, const int8_t* wq,
                                 const uint16_t* w_scale, int N, float* y,
                                 int32_t* partials_debug, void* stream);

/*
 * act_quant_w4a8_linear_ws / act_quant_w8a8_linear_ws -- the fused calls
 * with a workspace: for a verify batch (M >= 2, the MFMA forms; or a row
 * longer than the single-row fused kernel takes) the rows are rotated and
 * quantized inside the linear's own launch, once: workgroup m (m < M) writes
 * row m into xq / x_scale before it requests any weights, and every
 * workgroup requests its first weight batch, then waits for all M rows before
 * it reads activation codes.  No launch of its own for the quantization,
 * for callers that want one launch per linear; on MI355X the hand-off inside
 * the launch (about 5 us from launch to the last row visible at M = 16,
 * K = 4096) measured slower than the two-launch path.  [KT "Producing several tokens from one model pass": one
 * verification pass runs the linears on 16-32 candidate rows; "Why
 * batch-one decoding is memory-bound": the pass should cost its bytes.]
 * Arguments, outputs and errors as for act_quant_w4a8_linear /
 * act_quant_w8a8_linear (32-wide W4 groups at M > 2 keep the separate
 * quantization launch), plus:
 *  workspace  SVG_LINEAR_WORKSPACE_BYTES of device memory, 256-byte aligned,
 *             zero-filled before its first use; each call leaves it zero-
 *             filled again except word 3, a sticky flag set (to 1) if a
 *             bounded wait of the launch ever gave up (then y is
 *             undefined).  Calls that may overlap need different workspaces.
 *  Errors: SVG_EINVAL for a null workspace, SVG_EALIGN for a misaligned one.
 */
#define SVG_LINEAR_WORKSPACE_BYTES 256
svg_status act_quant_w4a8_linear_ws(const float* X, int M, int K, const int8_t* signs, int block,
                                    int8_t* xq, float* x_scale, const uint8_t* wq, const uint16_t* w_scale,
                                    const void* w_zero, int fmt, int group, int N, float* y,
                                    int32_t* partials_debug, void* workspace, void* stream);
svg_status act_quant_w8a8_linear_ws(const float* X, int M, int K, const int8_t* signs, int block,
                                    int8_t* xq, float* x_scale, const int8_t* wq, const uint16_t* w_scale,
                                    int N, float* y, int32_t* partials_debug, void* workspace, void* stream);

/*
 * tree_accept_greedy -- greedy acceptance of a verified draft tree.
 * [KT "Producing several tokens from one model pass": the main model checks the
 *  drafted positions together, keeps the valid prefix and continues from the
 *  first rejected position with its own token -- five drafted tokens of which
 *  it agrees with the first four advance the sequence by five; "Issue with
 *  parallel draft generation": over a tree of drafts it accepts the longest
 *  valid path.  The pages give no procedure beyond that; the readings below
 *  are this library's.]
 *
 *  logits    [T][V] fp32, row-major, 4-byte aligned: row i is the target
 *            model's prediction for the position after node i (the verify
 *            pass's output rows, in the order of its batch).
 *  T         nodes, 1 <= T <= SVG_TREE_MAX_NODES.  Node 0 is the root: the
 *            last token already in the sequence.
 *  V         vocabulary size, >= 1.
 *  parent    [T] int32: parent[0] = -1, and 0 <= parent[i] < i for i >= 1.
 *  draft     [T] int32: the token of each node (draft[0] is not read).
 *  target    OUTPUT [T] int32: the target's greedy choice at each node, the
 *            index of the largest logit of its row, the smallest index among
 *            equal maxima (NaN logits are outside the contract).
 *  path      OUTPUT [T] int32: the accepted nodes below the root, root side
 *            first, then -1.  Node i >= 1 is valid when its parent is valid and
 *            draft[i] == target[parent[i]] (the root is valid); the accepted
 *            path is the root path of the deepest valid node, the one with the
 *            smallest index among equally deep ones.
 *  emit      OUTPUT [T] int32: the emitted tokens -- the drafted tokens along
 *            the path, then the target's choice at its last node -- then -1.
 *  n_emit    OUTPUT [1] int32: the number of emitted tokens (path length + 1);
 *            -1 if parent[] breaks the rule above, and then path and emit are
 *            all -1 (the device checks the tree; the host never reads it).
 *  workspace SVG_TREE_WORKSPACE_BYTES of device memory, 8-byte aligned,
 *            zero-filled by the caller before its first use; every call leaves
 *            it zero-filled again.  Calls that may run at the same time must
 *            use different workspaces.
 *
 *  One launch: the logits stream once (T * V * 4 bytes); the workgroup that
 *  finishes last reads the row maxima and walks the tree.
 *  Errors: SVG_EINVAL for a null pointer, T < 1 or V < 1; SVG_EUNSUPPORTED for
 *  T > SVG_TREE_MAX_NODES or V > 2^30; SVG_EALIGN for logits, parent, draft
 *  or an output not 4-byte aligned, or workspace not 8-byte aligned.
 */
enum { SVG_TREE_MAX_NODES = 32, SVG_TREE_WORKSPACE_BYTES = 512 };
svg_status tree_accept_greedy(const float* logits, int T, int V, const int32_t* parent,
                              const int32_t* draft, int32_t* target, int32_t* path, int32_t* emit,
                              int32_t* n_emit, void* workspace, void* stream);

/*
 * tree_accept_greedy_static -- tree_accept_greedy without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid hipMalloc).  It allocates nothing: the
 * workspace is the library's own static device array of
 * SVG_TREE_WORKSPACE_BYTES (512) bytes, one per device, held until the process
 * ends.  The first call on a device looks its address up and zero-fills it
 * with a small kernel enqueued on `stream` ahead of the call's own kernel;
 * every call leaves it zero-filled again.  All calls on one device share it:
 * calls that may overlap on one device (other streams, other threads) race
 * and must not be made; use tree_accept_greedy with separate workspaces then.
 *  Arguments and outputs as for tree_accept_greedy.  T above
 *  SVG_TREE_MAX_NODES (32), the limit the array is sized for, is
 *  SVG_EUNSUPPORTED; a failure to find the array on the current device is
 *  SVG_EHIP.
 */
svg_status tree_accept_greedy_static(const float* logits, int T, int V, const int32_t* parent,
                                     const int32_t* draft, int32_t* target, int32_t* path,
                                     int32_t* emit, int32_t* n_emit, void* stream);

/*
 * tree_deltanet_verify, tree_deltanet_commit -- a fixed-state recurrent layer
 * over a draft tree, without restoring state.
 * [KT "Verifying a draft tree without restoring model state": a Gated
 *  DeltaNet layer folds the past into a fixed-size state that every accepted
 *  token changes; verification computes what every branch needs without
 *  touching the live state, and only the accepted tokens' updates are applied
 *  once the path is chosen.  The pages give no equations: the recurrence is
 *  the gated delta rule of the Gated DeltaNet publication.]
 *
 *  Per head, a state S of dv x dk fp32 values; per token a query q and a key
 *  k (dk values, the key of unit length), a value v (dv), a decay gate alpha
 *  in (0, 1] and a write strength beta in [0, 1]:
 *      S' = alpha * S (I - beta k k^T) + beta v k^T,     o = S' q.
 *  The tree is that of tree_accept_greedy (node 0 the root, parent[i] < i);
 *  the root is the last token of the sequence, not yet through the layer, so
 *  node i's state is the live state advanced along its root path, root first.
 *
 *  state   fp32 [H][dv][dk], 16-byte aligned: the live state (verify reads
 *          it only; commit updates it in place).
 *  q, k    fp32 [T][H][dk], 16-byte aligned.     v  fp32 [T][H][dv].
 *  alpha, beta  fp32 [T][H].                     parent  int32 [T].
 *  out     OUTPUT fp32 [T][H][dv]: o of every node (verify).  A node whose
 *          root path breaks the tree rule gets NaN.
 *  path, n_emit  commit's accepted path as tree_accept_greedy wrote it: the
 *          state advances by the root and path[0 .. n_emit - 2]; with
 *          n_emit < 1 or a node outside [1, T) the state is left as it was.
 *  T <= SVG_TREE_MAX_NODES; H >= 1; dk in {64, 128}, dv in {64, 128, 256}.  fp32 arithmetic with fused
 *  multiply-adds (the order of the sums differs from a plain loop: results
 *  are close to an exact computation, not bit-identical to one).
 *  One launch each.  Errors: SVG_EINVAL for a null pointer or T, H < 1;
 *  SVG_EUNSUPPORTED for T > 32, H > 65535 or another head size; SVG_EALIGN.
 */
svg_status tree_deltanet_verify(const float* state, const float* q, const float* k, const float* v,
                                const float* alpha, const float* beta, const int32_t* parent, int T,
                                int H, int dk, int dv, float* out, void* stream);
svg_status tree_deltanet_commit(float* state, const float* k, const float* v, const float* alpha,
                                const float* beta, const int32_t* path, const int32_t* n_emit, int T,
                                int H, int dk, int dv, void* stream);

/*
 * One pass of dependent W4A8 linears in ONE persistent launch.
 * [KT "Why batch-one decoding is memory-bound": a pass streams every weight
 *  once, so its time is bytes / bandwidth only if the weight stream never
 *  pauses; "How Uzu optimizes bytes and tokens per pass": activations are
 *  rotated and quantized on the fly; "Producing several tokens from one model
 *  pass": the verify pass runs the same linears on 16-32 candidate rows.]
 *
 * A pass is a list of steps, each act_quant_w4a8_linear on its own fp32 input
 * rows X (M rows, shared M).  With `after` set, a step's X is read only once
 * every earlier step has finished and its y is visible device-wide (y may be,
 * or feed, a later step's X); the launch keeps the weight stream going across
 * those waits by loading later steps' weights (which depend on nothing) ahead
 * of the activations.  Results are bit-identical in xq / x_scale / partials
 * to the single calls, and y agrees within fp32 summation order.
 *
 *  svg_pass_step   X, signs, xq, x_scale, wq, w_scale, w_zero, y,
 *                  partials_debug as for act_quant_w4a8_linear (same layouts,
 *                  same alignment); N >= 1 rows; K with K % 32 == 0,
 *                  K % group == 0, K % block == 0, K <= 12288; after: 0 or 1.
 *  svg_pass_plan   validates every step on the host and writes the pass's
 *                  device image to plan_host (host memory, info->plan_bytes;
 *                  NULL: validate and size only); the caller copies it to
 *                  device memory (8-byte aligned) once and may run it any
 *                  number of times.  All steps share M (1..16), fmt
 *                  (SVG_W4_ASYM_Z4 or _Z16), group (64 or 128) and block.
 *                  Fills *info (sizes included).
 *  svg_pass_run    enqueues the pass: one launch of one 1024-thread
 *                  workgroup per compute unit.  plan: the uploaded image;
 *                  info: as filled by svg_pass_plan; workspace:
 *                  info->workspace_bytes of device memory, 256-byte aligned,
 *                  zero-filled before first use; each run leaves its counters
 *                  zero-filled again, so it is reused as it is.  Word 0 is a
 *                  sticky flag the launch sets (to 1) if one of its bounded
 *                  waits ever gave up (then the outputs are undefined); it
 *                  needs every workgroup resident at once, i.e. no other
 *                  work on the device while it runs.  Runs that may overlap
 *                  need different workspaces.  The step table's pointers are
 *                  baked into the image: buffers must stay where they were.
 *  Errors: SVG_EINVAL / SVG_EUNSUPPORTED / SVG_EALIGN as for the single
 *  calls, plus SVG_EUNSUPPORTED for nsteps < 1, M > 16, group 32, K > 12288
 *  or a device with fewer than 8 compute units; svg_pass_run checks info
 *  against its own limits only (the image is trusted).
 */
typedef struct svg_pass_step {
    const float* X;
    const int8_t* signs;
    int8_t* xq;
    float* x_scale;
    const uint8_t* wq;
    const uint16_t* w_scale;
    const void* w_zero;
    float* y;
    int32_t* partials_debug;
    int N, K;
    int after;
} svg_pass_step;

typedef struct svg_pass_info {
    int nsteps, M, fmt, group, block;
    uint64_t plan_bytes, workspace_bytes;
} svg_pass_info;

svg_status svg_pass_plan(const svg_pass_step* steps, int nsteps, int M, int fmt, int group, int block,
                         void* plan_host, uint64_t plan_host_bytes, svg_pass_info* info);
svg_status svg_pass_run(const void* plan, const svg_pass_info* info, void* workspace, void* stream);

/*
 * Layout conversions between the canonical row-major arrays and the storage
 * the kernels read.  [KT "How Uzu optimizes bytes and tokens per pass": 4-bit
 * asymmetric codes with a scale and zero per group, 8-bit symmetric codes
 * with one scale per row, 8-bit activations -- the pages fix no layout; the
 * canonical one is the plainest row-major reading.]
 *
 * Canonical arrays (device memory, owned by the caller):
 *   W4 codes    [N][K/2] bytes: code (n, k) in byte n*K/2 + k/2, low nibble
 *               for even k, high nibble for odd k
 *   W4 scales   [N][K/group] fp16 (bit patterns)
 *   fp16 zeros  [N][K/group] fp16 (SVG_W4_ASYM_Z16; integer values 0..15)
 *   4-bit zeros [N][ceil(K/group/2)] bytes: zero (n, j) in byte
 *               n*ceil(K/group/2) + j/2, low nibble for even j (SVG_W4_ASYM_Z4)
 *   W8 codes    [N][K] int8;  W8 scales [N] fp16 (zero: NULL)
 *   act codes   [M][K] int8
 *
 *  svg_import_weights  canonical (codes, scale, zero) -> storage (wq, w_scale,
 *                      w_zero, sized by svg_weight_sizes; padding written 0).
 *                      The result is what rht_rotate_weights writes for the
 *                      same codes, scales and zeros.
 *  svg_export_weights  storage -> canonical (the inverse on the real rows
 *                      and groups).
 *  svg_import_act_codes  [M][K] rows -> xq in the 32-k slab layout of a
 *                      buffer of M rows (as act_rht_quant_i8 writes it).
 *  svg_export_act_codes  slab xq of M rows -> [M][K] rows.
 * Asynchronous on `stream`; pure data movement (no rotation, no rounding).
 * Errors (checked before any launch, outputs untouched): SVG_EINVAL for N, M
 * < 0, K <= 0 or a null required pointer (W4: zero and w_zero required);
 * SVG_EUNSUPPORTED for an unknown fmt, K % 32 != 0, a W4 group not in {32,
 * 64, 128} or not dividing K, K > 2^24, storage of 4 GiB or more, M*K >= 2^34;
 * SVG_EALIGN for wq or xq below 16 bytes, w_scale / fp16 w_zero below 4,
 * canonical fp16 arrays below 2, activation rows below 4.  Inputs and outputs
 * must not overlap.
 */
svg_status svg_import_weights(int fmt, int group, int N, int K, const void* codes, const uint16_t* scale,
                              const void* zero, void* wq, uint16_t* w_scale, void* w_zero, void* stream);
svg_status svg_export_weights(int fmt, int group, int N, int K, const void* wq, const uint16_t* w_scale,
                              const void* w_zero, void* codes, uint16_t* scale, void* zero, void* stream);
svg_status svg_import_act_codes(const int8_t* rows, int M, int K, int8_t* xq, void* stream);
svg_status svg_export_act_codes(const int8_t* xq, int M, int K, int8_t* rows, void* stream);

/* Text of the last error on the calling thread ("" after a successful call);
 * valid until the next call on this thread. */
const char* svg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SVGEMM_H */
