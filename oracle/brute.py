"""Brute-force checks for tiny inputs, in pure Python (TEST INFRASTRUCTURE).

Independent of svg_oracle.py: nothing here is imported from it.  These are the
textbook definitions written out with explicit loops, used by the tests to pin
the oracle:

* the Hadamard matrix by Sylvester's doubling, H_1 = [1], H_2n = [[H, H],
  [H, -H]] (no popcount formula);
* the rotation as an explicit matrix-vector product H . diag(s) . x per block of
  32, in exact integer (or Fraction) arithmetic;
* the integer contraction of the W4A8 and W8A8 linears as plain triple loops;
* the quantizers' rounding decisions on tiny rows and groups, every binary32
  operation done exactly on Fractions and rounded to binary32 / binary16 by
  integer code, and the butterfly one pair at a time in the same arithmetic.

Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
(blog.dailydoseofds.com), section "How Uzu optimizes bytes and tokens per
pass": the transform mixes each block of 32 with a +/-1 Hadamard after random
sign flips, both sides of the matmul are integers, activations take 8 bits on
the fly, Medium weights 4-bit asymmetric codes and Large weights 8-bit
symmetric ones.
"""
from __future__ import annotations


def sylvester(n: int):
    """Hadamard matrix of order n (a power of two) by Sylvester doubling, as a
    list of lists of Python ints."""
    H = [[1]]
    while len(H) < n:
        top = [row + row for row in H]
        bot = [row + [-v for v in row] for row in H]
        H = top + bot
    if len(H) != n:
        raise ValueError("n must be a power of two")
    return H


def rotate_row(x, signs, block=32):
    """u = blockdiag(H) . diag(signs) . x for one row (a list of exact
    numbers: ints or Fractions)."""
    H = sylvester(block)
    K = len(x)
    out = []
    for b0 in range(0, K, block):
        v = [signs[b0 + j] * x[b0 + j] for j in range(block)]
        for i in range(block):
            acc = 0
            for j in range(block):
                acc += H[i][j] * v[j]
            out.append(acc)
    return out


def w4_partials(qx, qw, z, group):
    """S[m][n][j] = sum_{k in group j} qx[m][k] * (qw[n][k] - z[n][j])."""
    M, K, N = len(qx), len(qx[0]), len(qw)
    G = K // group
    S = [[[0] * G for _ in range(N)] for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for j in range(G):
                acc = 0
                for k in range(j * group, (j + 1) * group):
                    acc += int(qx[m][k]) * (int(qw[n][k]) - int(z[n][j]))
                S[m][n][j] = acc
    return S


def w8_partials(qx, qw):
    """S[m][n] = sum_k qx[m][k] * qw[n][k]."""
    M, K, N = len(qx), len(qx[0]), len(qw)
    S = [[0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                acc += int(qx[m][k]) * int(qw[n][k])
            S[m][n] = acc
    return S


# ------------------------------------------------ exact IEEE rounding by hand
# The oracle decides every integer code with one fp32 operation (or an fp16
# conversion) followed by round-half-to-even.  The functions below redo those
# decisions from first principles: each operation is carried out exactly on
# rationals (Fraction) and then rounded to the nearest representable value by
# integer arithmetic, so no float64 intermediate (and no double rounding)
# enters.  Formats: binary32 (24-bit significand, smallest normal exponent
# -126) and binary16 (11-bit significand, smallest normal exponent -14);
# subnormals are kept.
from fractions import Fraction  # noqa: E402


def _round_to_format(x, prec: int, emin: int, emax: int) -> Fraction:
    """The value of the binary format (precision `prec`, exponents emin..emax)
    nearest to the exact rational x, ties to the even significand."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, emin) - (prec - 1))  # spacing of the format near a
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError("value beyond the format's finite range")
    return sign * r


def f32(x) -> Fraction:
    """Nearest binary32 value (round to nearest, ties to even)."""
    return _round_to_format(x, 24, -126, 127)


def f16(x) -> Fraction:
    """Nearest binary16 value (round to nearest, ties to even)."""
    return _round_to_format(x, 11, -14, 15)


def rne(x) -> int:
    """The integer nearest to the rational x, ties to the even integer."""
    x = Fraction(x)
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _clamp(v: int, lo: int, hi: int) -> int:
    return lo if v < lo else (hi if v > hi else v)


def fwht_f32(block_vals):
    """The unnormalised Walsh-Hadamard butterfly of one block (a list of
    binary32 values as Fractions; length a power of two), one pair at a time:
    stages h = 1, 2, 4, ... in ascending order, and at each stage the pair
    (v[i], v[i+h]) with bit h of i clear becomes (v[i] + v[i+h], v[i] - v[i+h]),
    each result rounded to binary32 on its own."""
    v = [Fraction(a) for a in block_vals]
    n = len(v)
    h = 1
    while h < n:
        for i in range(n):
            if i & h:
                continue
            a, b = v[i], v[i + h]
            v[i], v[i + h] = f32(a + b), f32(a - b)
        h *= 2
    return v


def act_quant_row_exact(u, block: int = 32):
    """Per-token symmetric int8 codes of one rotated row u (binary32 values as
    Fractions), every decision an exactly rounded binary32 operation:
    amax = max |u|; sigma = fl32(amax / 127); code = clamp(rne(fl32(u / sigma)),
    -127, 127), all zero for a zero row; stored scale fl32(sigma / block) (exact
    unless it falls below binary32's normal range).  Returns (codes, scale) as
    (list of int, Fraction)."""
    amax = max(abs(Fraction(a)) for a in u)
    if amax == 0:
        return [0] * len(u), Fraction(0)
    sigma = f32(amax / 127)
    codes = [_clamp(rne(f32(Fraction(a) / sigma)), -127, 127) for a in u]
    return codes, f32(sigma / block)


def w4_group_exact(u):
    """4-bit asymmetric codes of one group of rotated weights u (binary32
    values as Fractions): lo = min(0, min u), hi = max(0, max u);
    s = fl16(fl32(fl32(hi - lo) / 15)), 1 when that is 0; zero point
    z = clamp(rne(fl32(-lo / s)), 0, 15) (a 4-bit unsigned value);
    code = clamp(rne(fl32(u / s)) + z, 0, 15).  Returns (codes, s, z)."""
    vals = [Fraction(a) for a in u]
    lo = min(Fraction(0), min(vals))
    hi = max(Fraction(0), max(vals))
    s = f16(f32(f32(hi - lo) / 15))
    if s == 0:
        s = Fraction(1)
    z = _clamp(rne(f32(-lo / s)), 0, 15)
    codes = [_clamp(rne(f32(a / s)) + z, 0, 15) for a in vals]
    return codes, s, z


def w8_row_exact(u):
    """8-bit symmetric codes of one rotated weight row u (binary32 values as
    Fractions): s = fl16(fl32(max |u| / 127)), 1 when that is 0;
    code = clamp(rne(fl32(u / s)), -127, 127).  Returns (codes, s)."""
    vals = [Fraction(a) for a in u]
    a = max(abs(v) for v in vals)
    s = f16(f32(a / 127))
    if s == 0:
        s = Fraction(1)
    return [_clamp(rne(f32(v / s)), -127, 127) for v in vals], s
