"""CPU oracle of the RHT + W4A8 / W8A8 quantized linear (numpy, plain and slow).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path.

Sources.  [KT] is the page "Karpathy's Trick for Faster Local LLMs Finally Has
Proper Tooling" (blog.dailydoseofds.com); [VM] is the page "Giới thiệu
vllm-metal: Phục vụ đồng thời trên Apple Silicon" (gpuhub.net).  Each function
names the section it follows.

What the pages fix, and the readings taken where they are silent:

* [KT "How Uzu optimizes bytes and tokens per pass"]: weights are rotated by a
  block-diagonal random Hadamard transform before quantization -- random sign
  flips first, then a +/-1 Hadamard with one overall scale on each block of 32
  values; the transform is exactly reversible, so apart from rounding the
  layer computes the same thing.  Medium weights are 4-bit asymmetric
  integers, Large weights 8-bit symmetric; activations are quantized to 8 bits
  on the fly and the matmul is integer x integer.  The transform block and the
  quantization group are independent sizes.
* Readings (the pages give no formula): the Sylvester Hadamard in natural
  order; both operands of the contraction (weight rows and activation rows)
  are rotated by the same signs and blocks along K, which is what keeps the
  product unchanged; the transform is applied unnormalised (+/-1 entries) and
  the combined overall scale 1/sqrt(32) * 1/sqrt(32) = 2^-5 is folded exactly
  into the activation scale; the butterfly runs stages h = 1, 2, 4, 8, 16 in
  that order, every add/sub one fp32 round-to-nearest-even operation; per-token
  symmetric int8 activations with codes in [-127, 127]; min/max asymmetric W4
  per group along K with the range widened to contain 0, fp16 scale, integer
  zero point clamped to [0, 15] (a 4-bit unsigned value); per-output-row symmetric W8 with fp16 scale.
* A second transform block, 64 (the width of one CDNA wave, where the pages'
  32 is the width of the SIMD group of the hardware they target), is a
  variant: the same butterfly with one more stage (h = 32) and the combined
  overall scale 1/64 folded into the activation scale.  Block and group stay
  independent.
* Where floating point decides an integer code, the decision is taken in fp32
  (the kernels' precision) with IEEE division and round-half-to-even, so the
  codes are unique.  The reference output is then formed in fp64 from exact
  integer partial sums.

Contract: inputs are finite, and weights small enough that every fp16 scale
is finite (|W| < 4.9e5).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
F32 = np.float32


# ------------------------------------------------------------ the transform
BLOCKS = (32, 64)  # 32: the pages' block; 64: the wave-wide variant (one CDNA wave)


def hadamard(block: int = BLOCK) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j), i, j in 0..block-1: the Sylvester-ordered
    Hadamard matrix, entries +/-1 [KT "How Uzu optimizes bytes and tokens per
    pass": a Hadamard matrix holds only +1 and -1 plus one overall scale]."""
    i = np.arange(block)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def hadamard32() -> np.ndarray:
    """The order-32 matrix of the pages' block size."""
    return hadamard(32)


def fwht(v: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of every aligned block of `block`
    values along the last axis, in v's dtype (fp32 or fp64).

    Stage order h = 1, 2, 4, ..., block/2; at stage h every index i of a block
    with (i & h) == 0 maps the pair (v[i], v[i+h]) to (v[i] + v[i+h],
    v[i] - v[i+h]), each a single rounded operation.  In exact arithmetic the
    result is H @ block with H = hadamard(block) [KT "How Uzu optimizes bytes
    and tokens per pass": each block is mixed on its own]."""
    if block not in BLOCKS:
        raise ValueError(f"block must be one of {BLOCKS}")
    v = np.array(v, copy=True)
    shape = v.shape
    if shape[-1] % block:
        raise ValueError(f"last axis must be a multiple of {block}")
    b = v.reshape(-1, shape[-1] // block, block)
    h = 1
    while h < block:
        lo = [i for i in range(block) if not i & h]
        hi = [i + h for i in lo]
        a = b[:, :, lo]
        c = b[:, :, hi]
        b[:, :, lo] = a + c
        b[:, :, hi] = a - c
        h *= 2
    return b.reshape(shape)


def fwht32(v: np.ndarray) -> np.ndarray:
    """The transform with the pages' block of 32 (stages h = 1, 2, 4, 8, 16)."""
    return fwht(v, 32)


def rht(r: np.ndarray, signs: np.ndarray, dtype=F32, block: int = BLOCK) -> np.ndarray:
    """Block-diagonal random Hadamard transform of the rows of r along the last
    axis: the +/-1 sign flip first, then the block Hadamard
    [KT "How Uzu optimizes bytes and tokens per pass": random sign flips are
    applied before the mixing].  Unnormalised: u = H_B . diag(signs) . r."""
    r = np.asarray(r, dtype=dtype)
    s = np.asarray(signs).astype(dtype)
    if r.shape[-1] != s.shape[-1]:
        raise ValueError("signs length must equal K")
    return fwht32(r * s) if block == 32 else fwht(r * s, block)


# ------------------------------------------------- activation quantization
def act_quant_i8(u: np.ndarray, block: int = BLOCK):
    """Per-token symmetric int8 quantization of rotated activation rows u[M, K]
    (fp32) [KT "How Uzu optimizes bytes and tokens per pass": activations are
    quantized to 8 bits on the fly].

    amax = max_k |u|; sigma = amax / 127 (fp32); q = clamp(rint(u / sigma),
    -127, 127); a zero row gives q = 0.  Returns (q int8 [M, K], scale fp32 [M])
    where scale = sigma / block also carries the transform's overall scale
    (1/sqrt(block) on each operand; 2^-5 for the pages' 32), so that
    x . w  ~=  scale[m] * sum_k q[m, k] * (dequantized rotated weight)."""
    u = np.asarray(u, dtype=F32)
    amax = np.max(np.abs(u), axis=-1)
    sigma = amax / F32(127)
    safe = np.where(amax > 0, sigma, F32(1))
    q = np.clip(np.rint(u / safe[..., None]), -127, 127)
    q = np.where(amax[..., None] > 0, q, F32(0)).astype(np.int8)
    # a power-of-two factor: exact, except where sigma / block falls below the
    # normal range and rounds like any fp32 product
    scale = (sigma * F32(1.0 / block)).astype(F32)
    return q, scale


# ------------------------------------------------------ weight quantizers
def quant_w4(u: np.ndarray, group: int):
    """4-bit asymmetric integer quantization ("Medium") of rotated weight rows
    u[N, K] (fp32), one (scale, zero) pair per `group` consecutive values along K
    [KT "How Uzu optimizes bytes and tokens per pass": Medium is 4-bit
    asymmetric integer quantization; every value of a group shares one scale].

    Per group: lo = min(0, min u), hi = max(0, max u); s = fp16(rne((hi - lo) /
    15)), replaced by 1.0 if zero; z = clamp(rint(-lo / s), 0, 15) -- the zero
    point is an unsigned 4-bit integer, and -lo / s can pass 15 when s lands in
    fp16's subnormal range, where its relative rounding is coarse;
    q = clamp(rint(u / s) + z, 0, 15).  Returns (q uint8 [N, K] in 0..15,
    s fp16 [N, K/group], z uint8 [N, K/group])."""
    u = np.asarray(u, dtype=F32)
    N, K = u.shape
    if K % group:
        raise ValueError("K must be a multiple of the group")
    ug = u.reshape(N, K // group, group)
    lo = np.minimum(F32(0), ug.min(axis=-1))
    hi = np.maximum(F32(0), ug.max(axis=-1))
    s = ((hi - lo) / F32(15)).astype(np.float16)
    s = np.where(s == 0, np.float16(1.0), s).astype(np.float16)
    s32 = s.astype(F32)
    z = np.clip(np.rint(-lo / s32), 0, 15)
    q = np.clip(np.rint(ug / s32[..., None]) + z[..., None], 0, 15)
    return q.reshape(N, K).astype(np.uint8), s, z.astype(np.uint8)


def quant_w8(u: np.ndarray):
    """8-bit symmetric quantization ("Large") of rotated weight rows u[N, K],
    one fp16 scale per output row [KT "How Uzu optimizes bytes and tokens per
    pass": Large is 8-bit symmetric quantization].

    a = max_k |u|; s = fp16(rne(a / 127)), replaced by 1.0 if zero;
    q = clamp(rint(u / s), -127, 127).  Returns (q int8 [N, K], s fp16 [N])."""
    u = np.asarray(u, dtype=F32)
    a = np.max(np.abs(u), axis=-1)
    s = (a / F32(127)).astype(np.float16)
    s = np.where(s == 0, np.float16(1.0), s).astype(np.float16)
    q = np.clip(np.rint(u / s.astype(F32)[:, None]), -127, 127).astype(np.int8)
    return q, s


# ----------------------------------------------------- integer contraction
def w4_group_partials(qx: np.ndarray, q: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    """S[m, n, j] = sum over k in group j of qx[m, k] * (q[n, k] - z[n, j]),
    exact in int64 [KT "How Uzu optimizes bytes and tokens per pass": with both
    sides stored as integers the matmul runs on the int8 matrix path]."""
    M, K = qx.shape
    N = q.shape[0]
    G = K // group
    xg = np.asarray(qx, dtype=np.int64).reshape(M, G, group)
    wg = np.asarray(q, dtype=np.int64).reshape(N, G, group) - np.asarray(z, dtype=np.int64)[:, :, None]
    return np.einsum("mjk,njk->mnj", xg, wg)


def w8_partials(qx: np.ndarray, q: np.ndarray) -> np.ndarray:
    """S[m, n] = sum_k qx[m, k] * q[n, k], exact in int64."""
    return np.einsum("mk,nk->mn", np.asarray(qx, dtype=np.int64), np.asarray(q, dtype=np.int64))


def w4a8_output(x_scale: np.ndarray, S: np.ndarray, s: np.ndarray) -> np.ndarray:
    """y[m, n] = x_scale[m] * sum_j s[n, j] * S[m, n, j], in fp64."""
    return np.asarray(x_scale, np.float64)[:, None] * np.einsum(
        "mnj,nj->mn", S.astype(np.float64), np.asarray(s, np.float64))


def w8a8_output(x_scale: np.ndarray, S: np.ndarray, s: np.ndarray) -> np.ndarray:
    """y[m, n] = x_scale[m] * s[n] * S[m, n], in fp64."""
    return (np.asarray(x_scale, np.float64)[:, None] * np.asarray(s, np.float64)[None, :]
            * S.astype(np.float64))


# ------------------------------------------------------------ whole layer
def prepare_w4(W: np.ndarray, signs: np.ndarray, group: int, block: int = BLOCK) -> dict:
    """Offline: rotate the fp32 weight rows, then quantize them as Medium."""
    u = rht(W, signs, F32, block)
    q, s, z = quant_w4(u, group)
    return dict(q=q, s=s, z=z, group=group, block=block)


def prepare_w8(W: np.ndarray, signs: np.ndarray, block: int = BLOCK) -> dict:
    """Offline: rotate the fp32 weight rows, then quantize them as Large."""
    q, s = quant_w8(rht(W, signs, F32, block))
    return dict(q=q, s=s, block=block)


def quant_acts(x: np.ndarray, signs: np.ndarray, block: int = BLOCK):
    """Online: rotate the activation rows with the weights' signs, then
    quantize them per token to int8."""
    return act_quant_i8(rht(x, signs, F32, block), block)


def linear_w4(x: np.ndarray, signs: np.ndarray, w: dict):
    """One W4A8 linear: returns (y fp64 [M, N], S int64 [M, N, G], qx, x_scale).
    The activations take the weights' transform block."""
    qx, sx = quant_acts(x, signs, w.get("block", BLOCK))
    S = w4_group_partials(qx, w["q"], w["z"], w["group"])
    return w4a8_output(sx, S, w["s"]), S, qx, sx


def linear_w8(x: np.ndarray, signs: np.ndarray, w: dict):
    """One W8A8 linear: returns (y fp64 [M, N], S int64 [M, N], qx, x_scale)."""
    qx, sx = quant_acts(x, signs, w.get("block", BLOCK))
    S = w8_partials(qx, w["q"])
    return w8a8_output(sx, S, w["s"]), S, qx, sx


# ------------------------------------------------------- byte accounting
def linear_bytes(M: int, N: int, K: int, fmt: str, group: int) -> int:
    """Algorithmic bytes one linear must touch once: packed weight codes, their
    scales and zeros, the int8 activation codes and scales in, fp32 outputs out
    [KT "Why batch-one decoding is memory-bound": every pass streams every
    weight once].  fmt is "w4_z4", "w4_z16" or "w8"."""
    if fmt == "w8":
        wbytes = N * K + 2 * N
    else:
        G = K // group
        zbytes = N * ((G + 1) // 2) if fmt == "w4_z4" else 2 * N * G
        wbytes = N * K // 2 + 2 * N * G + zbytes
    return wbytes + M * K + 4 * M + 4 * M * N


def passes_per_second(bandwidth_bytes_per_s: float, bytes_per_pass: float) -> float:
    """Byte-bound ceiling on model passes per second: bandwidth / bytes read per
    pass [KT "Why batch-one decoding is memory-bound"]."""
    return bandwidth_bytes_per_s / bytes_per_pass


# -------------------------------------------------------------- parity metric
def output_error(y: np.ndarray, y_ref: np.ndarray, floor: float = 1e-3):
    """Error of fp32 outputs y against the fp64 reference.

    Returns (elementwise, rownorm, excluded): elementwise is max |y - y_ref| /
    |y_ref| over elements with |y_ref| >= floor * max_n |y_ref[m, n]| of their
    row; rownorm is max_m ||y_m - y_ref_m||_inf / ||y_ref_m||_inf; excluded is
    the number of elements below the floor (which only enter rownorm)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    rowmax = np.max(np.abs(y_ref), axis=-1, keepdims=True)
    err = np.abs(y - y_ref)
    mask = np.abs(y_ref) >= floor * rowmax
    mask &= rowmax > 0
    elem = float(np.max(np.where(mask, err / np.where(mask, np.abs(y_ref), 1.0), 0.0))) if y.size else 0.0
    rown = np.max(err, axis=-1) / np.where(rowmax[:, 0] > 0, rowmax[:, 0], 1.0)
    rown = np.where(rowmax[:, 0] > 0, rown, np.max(err, axis=-1))
    return elem, float(np.max(rown)) if y.size else 0.0, int(y.size - np.count_nonzero(mask))
