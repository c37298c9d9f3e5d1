"""Exact construction of the scaled Winograd transforms F(m, 3).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source: "Data-Free Group-Wise Fully Quantized Winograd Convolution via
Learnable Scales" (arXiv 2412.19867).
  * Appendix 7.1 "Standard Winograd transforms": from polynomial points
    (f_i, g_i) a Vandermonde matrix V_{a x b} has entry f_i^j * g_i^(b-1-j)
    in row i, column j (the printed matrix is garbled; this is its plain
    reading, with the point at infinity written (1, 0)).
  * "What carries the argument": B^T = S_B V^-T, G = S_G V, A^T = V^T S_A
    with diagonal S_A S_B S_G = I; only S_B and S_G are free.

Here V without a subscript means the square n x n matrix for B^T, the n x 3
matrix for G and the n x m matrix for A^T (n = m + 2). Every entry is an exact
rational; the fp32 / fp64 matrices handed to the fp pipelines are the exact
values rounded once, to nearest with ties to even.

Standard points (the pages take them from their reference [2] without printing
them; reading: the usual Toom-Cook choice):
  F(4,3): 0, 1, -1, 2, -2, inf
  F(6,3): 0, 1, -1, 2, -2, 1/2, -1/2, inf
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

INF = float("inf")


def standard_points(m: int) -> list[float]:
    if m == 2:
        return [0.0, 1.0, -1.0, INF]
    if m == 4:
        return [0.0, 1.0, -1.0, 2.0, -2.0, INF]
    if m == 6:
        return [0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, INF]
    raise ValueError(f"no standard points for m={m}")


def homogeneous(p: float) -> tuple[Fraction, Fraction]:
    """Finite p -> (p, 1); the point at infinity -> (1, 0)."""
    if math.isinf(p):
        return Fraction(1), Fraction(0)
    return Fraction(p), Fraction(1)


def vandermonde(points, cols: int) -> list[list[Fraction]]:
    """V[i][j] = f_i^j * g_i^(cols-1-j)   (0^0 = 1)."""
    rows = []
    for p in points:
        f, g = homogeneous(p)
        rows.append([f ** j * g ** (cols - 1 - j) for j in range(cols)])
    return rows


def inverse(a: list[list[Fraction]]) -> list[list[Fraction]]:
    """Exact inverse by Gauss-Jordan elimination over the rationals."""
    n = len(a)
    aug = [list(row) + [Fraction(int(i == j)) for j in range(n)] for i, row in enumerate(a)]
    for col in range(n):
        piv = next((r for r in range(col, n) if aug[r][col] != 0), None)
        if piv is None:
            raise ValueError("points are not distinct: Vandermonde matrix is singular")
        aug[col], aug[piv] = aug[piv], aug[col]
        p = aug[col][col]
        aug[col] = [v / p for v in aug[col]]
        for r in range(n):
            if r != col and aug[r][col] != 0:
                f = aug[r][col]
                aug[r] = [vr - f * vc for vr, vc in zip(aug[r], aug[col])]
    return [row[n:] for row in aug]


def matmul(a, b):
    return [[sum((a[i][k] * b[k][j] for k in range(len(b))), Fraction(0))
             for j in range(len(b[0]))] for i in range(len(a))]


def exact_transforms(m: int, points, s_b, s_g):
    """Exact (Bt [n][n], G [n][3], At [m][n]) for the given points and scales.

    Bt[i][k] = s_B[i] * (V_n^-1)[k][i]
    G[i][k]  = s_G[i] * V_{n x 3}[i][k]
    At[a][k] = V_{n x m}[k][a] * s_A[k],   s_A[k] = 1 / (s_B[k] s_G[k])
    """
    n = m + 2
    if len(points) != n or len(s_b) != n or len(s_g) != n:
        raise ValueError("need n = m + 2 points and scales")
    exact = lambda v: v if isinstance(v, Fraction) else Fraction(float(v))
    sb = [exact(v) for v in s_b]
    sg = [exact(v) for v in s_g]
    if any(v == 0 for v in sb + sg):
        raise ValueError("scales must be non-zero")
    vn = vandermonde(points, n)
    vinv = inverse(vn)
    vr = vandermonde(points, 3)
    vm = vandermonde(points, m)
    bt = [[sb[i] * vinv[k][i] for k in range(n)] for i in range(n)]
    gm = [[sg[i] * vr[i][k] for k in range(3)] for i in range(n)]
    sa = [1 / (sb[k] * sg[k]) for k in range(n)]
    at = [[vm[k][a] * sa[k] for k in range(n)] for a in range(m)]
    return bt, gm, at


def round_f32(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even), once.

    float32(float(q)) would round twice (to fp64, then to fp32) and can land on
    the wrong side of an fp32 midpoint; this rounds the exact value directly.
    Only normal-range results are needed here.
    """
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1); keep 24 significant bits
    scaled = a / Fraction(2) ** (e - 23)
    k = scaled.numerator // scaled.denominator
    rem = scaled - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    if e < -126 or e > 127:
        raise OverflowError("value outside the normal fp32 range")
    return np.float32(sign * float(k) * 2.0 ** (e - 23))


def round_f64(q: Fraction) -> float:
    """Nearest fp64 (CPython's int/int true division rounds correctly)."""
    return q.numerator / q.denominator


def transforms_f32(m, points, s_b, s_g):
    bt, gm, at = exact_transforms(m, points, s_b, s_g)
    conv = lambda mat: np.array([[round_f32(v) for v in row] for row in mat], dtype=np.float32)
    return conv(bt), conv(gm), conv(at)


def transforms_f64(m, points, s_b, s_g):
    bt, gm, at = exact_transforms(m, points, s_b, s_g)
    conv = lambda mat: np.array([[round_f64(v) for v in row] for row in mat], dtype=np.float64)
    return conv(bt), conv(gm), conv(at)
