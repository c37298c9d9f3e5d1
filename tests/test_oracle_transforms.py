"""Pins for the oracle's transform construction (oracle/transforms.py).

Nothing here retypes the construction: each check is against mathematics
that fixes the answer independently (matrix identities, the textbook
F(2,3) / F(4,3) matrices of Lavin & Gray, which the pages cite as their
reference [15], exact rational convolution, IEEE rounding).
"""
import random
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import transforms as T


# ---------------------------------------------------------------- rounding
def test_round_f32_matches_ieee_on_doubles():
    # an fp64 value is an exact rational; numpy's fp64 -> fp32 cast rounds it
    # once, to nearest even, so the two must agree bit for bit
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                           rng.uniform(-1, 1, 500)])
    for v in vals:
        assert T.round_f32(Fr(float(v))) == np.float32(v)


def test_round_f32_ties_and_double_rounding():
    one = Fr(1)
    ulp = Fr(1, 2 ** 23)
    assert T.round_f32(one + ulp / 2) == np.float32(1.0)               # tie -> even
    assert T.round_f32(one + 3 * ulp / 2) == np.float32(1 + 2.0 ** -22)  # tie -> even (up)
    # just above the tie by far less than an fp64 ulp: fp64 would round to the
    # tie and then to even (1.0); a single rounding goes up
    q = one + ulp / 2 + Fr(1, 2 ** 80)
    assert np.float32(float(q)) == np.float32(1.0)
    assert T.round_f32(q) == np.float32(1 + 2.0 ** -23)
    assert T.round_f32(-q) == -np.float32(1 + 2.0 ** -23)
    assert T.round_f32(Fr(0)) == 0


# ------------------------------------------------------ Vandermonde algebra
@pytest.mark.parametrize("m", [2, 4, 6])
def test_inverse_is_exact(m):
    n = m + 2
    for pts in (T.standard_points(m),
                [float(p) for p in random.Random(m).sample(range(-9, 10), n - 1)] + [T.INF]):
        V = T.vandermonde(pts, n)
        Vi = T.inverse(V)
        I = T.matmul(V, Vi)
        assert all(I[i][j] == (1 if i == j else 0) for i in range(n) for j in range(n))


def test_duplicate_points_rejected():
    with pytest.raises(ValueError):
        T.inverse(T.vandermonde([0.0, 1.0, 1.0, T.INF], 4))


def test_point_at_infinity_row():
    # homogeneous (1, 0): only the highest power survives
    V = T.vandermonde([T.INF], 5)
    assert V[0] == [0, 0, 0, 0, 1]


# ------------------------------------------------------ textbook matrices
LAVIN_F23 = dict(
    Bt=[[1, 0, -1, 0], [0, 1, 1, 0], [0, -1, 1, 0], [0, 1, 0, -1]],
    G=[[1, 0, 0], [Fr(1, 2), Fr(1, 2), Fr(1, 2)], [Fr(1, 2), Fr(-1, 2), Fr(1, 2)], [0, 0, 1]],
    At=[[1, 1, 1, 0], [0, 1, -1, -1]],
)
LAVIN_F43 = dict(
    Bt=[[4, 0, -5, 0, 1, 0], [0, -4, -4, 1, 1, 0], [0, 4, -4, -1, 1, 0],
        [0, -2, -1, 2, 1, 0], [0, 2, -1, -2, 1, 0], [0, 4, 0, -5, 0, 1]],
    G=[[Fr(1, 4), 0, 0], [Fr(-1, 6), Fr(-1, 6), Fr(-1, 6)], [Fr(-1, 6), Fr(1, 6), Fr(-1, 6)],
       [Fr(1, 24), Fr(1, 12), Fr(1, 6)], [Fr(1, 24), Fr(-1, 12), Fr(1, 6)], [0, 0, 1]],
    At=[[1, 1, 1, 1, 1, 0], [0, 1, -1, 2, -2, 0], [0, 1, 1, 4, 4, 0], [0, 1, -1, 8, -8, 1]],
)


def _corr_1d_exact(Bt, G, At, m):
    """1D check: At[(G g) .* (Bt d)] must equal sum_a g[a] d[k+a] exactly."""
    rnd = random.Random(5)
    n = m + 2
    for _ in range(20):
        d = [Fr(rnd.randint(-50, 50)) for _ in range(n)]
        g = [Fr(rnd.randint(-50, 50)) for _ in range(3)]
        u = [sum(Fr(G[i][a]) * g[a] for a in range(3)) for i in range(n)]
        v = [sum(Fr(Bt[i][k]) * d[k] for k in range(n)) for i in range(n)]
        y = [sum(Fr(At[a][i]) * u[i] * v[i] for i in range(n)) for a in range(m)]
        ref = [sum(g[a] * d[k + a] for a in range(3)) for k in range(m)]
        assert y == ref


@pytest.mark.parametrize("m,book", [(2, LAVIN_F23), (4, LAVIN_F43)])
def test_textbook_matrices_are_valid(m, book):
    _corr_1d_exact(book["Bt"], book["G"], book["At"], m)


@pytest.mark.parametrize("m,book,s_g,s_a", [
    (2, LAVIN_F23, [1, Fr(1, 2), Fr(1, 2), 1], [1, 1, 1, -1]),
    (4, LAVIN_F43, [Fr(1, 4), Fr(-1, 6), Fr(-1, 6), Fr(1, 24), Fr(1, 24), 1], [1] * 6),
])
def test_construction_reproduces_textbook(m, book, s_g, s_a):
    # the textbook triple is the Vandermonde construction for the standard
    # points with diagonal scales; S_B follows from S_A S_B S_G = I
    s_g = [Fr(v) for v in s_g]
    s_b = [1 / (Fr(a) * g) for a, g in zip(s_a, s_g)]
    bt, gm, at = T.exact_transforms(m, T.standard_points(m), s_b, s_g)
    assert bt == [[Fr(v) for v in r] for r in book["Bt"]]
    assert gm == [[Fr(v) for v in r] for r in book["G"]]
    assert at == [[Fr(v) for v in r] for r in book["At"]]


# ------------------------------------------------- exact 2D convolution
def _direct_2d(d, g, m):
    return [[sum(g[a][b] * d[i + a][j + b] for a in range(3) for b in range(3))
             for j in range(m)] for i in range(m)]


def _wino_2d(d, g, bt, gm, at, m):
    n = m + 2
    tr = lambda a: [list(r) for r in zip(*a)]
    U = T.matmul(T.matmul(gm, g), tr(gm))
    V = T.matmul(T.matmul(bt, d), tr(bt))
    Y = [[U[i][j] * V[i][j] for j in range(n)] for i in range(n)]
    return T.matmul(T.matmul(at, Y), tr(at))


@pytest.mark.parametrize("m", [4, 6])
@pytest.mark.parametrize("scales", ["identity", "rational", "fp32_random"])
def test_exact_winograd_equals_direct(m, scales):
    """The scale identity S_A S_B S_G = I: for any non-zero diagonal scales the
    exact Winograd tile equals the exact direct correlation."""
    n = m + 2
    rnd = random.Random(100 * m + len(scales))
    if scales == "identity":
        sb = sg = [Fr(1)] * n
    elif scales == "rational":
        sb = [Fr(rnd.choice([-1, 1]) * rnd.randint(1, 9), rnd.randint(1, 9)) for _ in range(n)]
        sg = [Fr(rnd.randint(1, 9), rnd.randint(1, 9)) for _ in range(n)]
    else:
        r = np.random.default_rng(m)
        sb = [Fr(float(v)) for v in np.exp(r.uniform(-.5, .5, n)).astype(np.float32)]
        sg = [Fr(float(v)) for v in np.exp(r.uniform(-.5, .5, n)).astype(np.float32)]
    bt, gm, at = T.exact_transforms(m, T.standard_points(m), sb, sg)
    for _ in range(3):
        d = [[Fr(rnd.randint(-20, 20)) for _ in range(n)] for _ in range(n)]
        g = [[Fr(rnd.randint(-20, 20)) for _ in range(3)] for _ in range(3)]
        assert _wino_2d(d, g, bt, gm, at, m) == _direct_2d(d, g, m)


def test_rounded_matrices_are_nearest():
    # fp32 entries are the exact values rounded once; fp64 likewise
    m = 6
    r = np.random.default_rng(3)
    sb = np.exp(r.uniform(-.5, .5, 8)).astype(np.float32)
    sg = np.exp(r.uniform(-.5, .5, 8)).astype(np.float32)
    ex = T.exact_transforms(m, T.standard_points(m), sb, sg)
    f32 = T.transforms_f32(m, T.standard_points(m), sb, sg)
    f64 = T.transforms_f64(m, T.standard_points(m), sb, sg)
    for e, a, b in zip(ex, f32, f64):
        for i, row in enumerate(e):
            for j, q in enumerate(row):
                # |fp32 - exact| <= half an fp32 ulp, and it is the closer neighbour
                x = a[i, j]
                err = abs(Fr(float(x)) - q)
                if q != 0:
                    up = Fr(float(np.nextafter(x, np.float32(np.inf))))
                    dn = Fr(float(np.nextafter(x, np.float32(-np.inf))))
                    assert err <= abs(up - q) and err <= abs(dn - q)
                else:
                    assert x == 0
                assert abs(Fr(float(b[i, j])) - q) <= abs(q) * Fr(1, 2 ** 53)
