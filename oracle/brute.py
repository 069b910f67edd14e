"""Brute-force checks for tiny inputs, in pure Python (TEST INFRASTRUCTURE).

Independent of svg_oracle.py: nothing here is imported from it.  These are the
textbook definitions written out with explicit loops, used by the tests to pin
the oracle:

* the Hadamard matrix by Sylvester's doubling, H_1 = [1], H_2n = [[H, H],
  [H, -H]] (no popcount formula);
* the rotation as an explicit matrix-vector product H . diag(s) . x per block of
  32, in exact integer (or Fraction) arithmetic;
* the integer contraction of the W4A8 and W8A8 linears as plain triple loops.

Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
(blog.dailydoseofds.com), section "How Uzu optimizes bytes and tokens per
pass": the transform mixes each block of 32 with a +/-1 Hadamard after random
sign flips, and both sides of the matmul are integers.
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
