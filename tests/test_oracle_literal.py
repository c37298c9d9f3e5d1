"""Pins for the oracle's literal input stage: B^T and the input patch
quantized, the input transform on integer codes, the factor "sqB sqB sqx"
(review page, Eqs. 14-16 as the minor comments name them) applied after it.

Each pin fixes the answer independently of the oracle's own code:
  - hand-derived codes of the textbook F(4,3) B^T under both granularities
    (including a half-way case that ties to even);
  - on integer-valued inputs and an integer B^T whose scales are exactly 1,
    the literal stage must reproduce the fp32 stage (pinned elsewhere) bit for
    bit, which fixes every index and transpose;
  - exact power-of-two scaling identities, which fix which scale multiplies
    which tap;
  - the geometric extent of a patch scale (which tiles a spike reaches);
  - an a-posteriori error bound against the exact fp64 transform.
"""
import numpy as np
import pytest

import oracle
from oracle import transforms as TR


def std_bt(m, prec="f32"):
    mk = TR.transforms_f32 if prec == "f32" else TR.transforms_f64
    n = m + 2
    return mk(m, TR.standard_points(m), np.ones(n, np.float32), np.ones(n, np.float32))[0]


def test_quant_bt_textbook_f43_hand_values():
    """B^T for the points 0, 1, -1, 2, -2, inf with S_B = I has rows
    (1, 0, -5/4, 0, 1/4, 0), (0, 2/3, 2/3, -1/6, -1/6, 0), ...,
    (0, 1/12, -1/24, -1/12, 1/24, 0), (0, 4, 0, -5, 0, 1). Codes are
    rint(b * 127 / absmax) worked out by hand."""
    Bt = std_bt(4)
    Bq, sB = oracle.quant_bt(Bt, rows=False)
    # one scale, absmax 5: 127/5 = 25.4 per unit
    exp_tensor = np.array([[25, 0, -32, 0, 6, 0],        # 25.4, -31.75, 6.35
                           [0, 17, 17, -4, -4, 0],       # 16.93, -4.23
                           [0, -17, 17, 4, -4, 0],
                           [0, -2, -1, 2, 1, 0],         # 2.117, 1.058
                           [0, 2, -1, -2, 1, 0],
                           [0, 102, 0, -127, 0, 25]])    # 101.6
    assert np.array_equal(Bq, exp_tensor)
    assert np.all(sB == np.float32(5) / np.float32(127))
    Bq, sB = oracle.quant_bt(Bt, rows=True)
    exp_rows = np.array([[102, 0, -127, 0, 25, 0],        # absmax 5/4: 1 -> 101.6, 1/4 -> 25.4
                         [0, 127, 127, -32, -32, 0],      # absmax 2/3: 1/6 -> 31.75
                         [0, -127, 127, 32, -32, 0],
                         [0, -127, -64, 127, 64, 0],      # absmax 1/12: 1/24 -> 63.5, tie to even
                         [0, 127, -64, -127, 64, 0],
                         [0, 102, 0, -127, 0, 25]])
    assert np.array_equal(Bq, exp_rows)
    absmax = np.array([1.25, 2 / 3, 2 / 3, 1 / 12, 1 / 12, 5], np.float32)
    assert np.array_equal(sB, absmax / np.float32(127))


def integer_bt(n, rng):
    """Integer B^T, every row holding +-127 once and small entries elsewhere,
    not symmetric, invertible in practice."""
    Bt = rng.integers(-2, 3, size=(n, n)).astype(np.float32)
    cols = rng.permutation(n)
    for i in range(n):
        Bt[i, cols[i]] = 127.0 if rng.random() < 0.5 else -127.0
    return Bt


def grid_input(N, Cin, H, W, G, rng):
    """Integers in [-3, 3], with the first channel of every group equal to
    127 everywhere: every (tile, group) patch has absmax 127, so its scale
    is 1 and its codes are the values."""
    x = rng.integers(-3, 4, size=(N, Cin, H, W)).astype(np.float32)
    x[:, ::G] = 127.0
    return x


@pytest.mark.parametrize("m,pad,rows", [(4, 1, False), (6, 1, True), (4, 0, True), (6, 2, False)])
def test_literal_equals_fp32_stage_on_grid(m, pad, rows):
    """With scales of exactly 1 every step is exact: the integer transform
    equals the fp32 transform (all partial sums are integers below 2^24, at
    most (127 + 2 (n-1))^2 * 127), so Vq and sV must be bit-identical to the
    fp32 stage on the same B^T."""
    rng = np.random.default_rng([11, m, pad, rows])
    n, G = m + 2, 16
    N, Cin, H, W = 2, 32, 2 * m + 1, 3 * m - 1
    Bt = integer_bt(n, rng)
    x = grid_input(N, Cin, H, W, G, rng)
    Bq, sB = oracle.quant_bt(Bt, rows)
    assert np.array_equal(Bq.astype(np.float32), Bt) and np.all(sB == 1.0)
    Vq, sV, xq, sx = oracle.stage1_int(m, x, pad, G, Bq, sB, keep=True)
    Vq0, sV0 = oracle.stage1(m, x, pad, G, Bt)
    assert np.all(sx == 1.0)
    assert np.array_equal(Vq, Vq0) and np.array_equal(sV, sV0)
    # the patch codes are the zero-padded patches themselves
    tH, tW, T = oracle.tiles(m, N, H, W, pad)
    xp = np.zeros((N, Cin, tH * m + 2, tW * m + 2), np.float32)
    hh, ww = min(H, tH * m + 2 - pad), min(W, tW * m + 2 - pad)
    xp[:, :, pad:pad + hh, pad:pad + ww] = x[:, :, :hh, :ww]
    for t in [0, T // 2, T - 1]:
        img, ty, tx = t // (tH * tW), t // tW % tH, t % tW
        patch = xp[img, :, ty * m:ty * m + n, tx * m:tx * m + n]
        assert np.array_equal(xq[t].astype(np.float32), patch)


@pytest.mark.parametrize("m", [4, 6])
def test_literal_power_of_two_scalings(m):
    """x * 2^a leaves every code unchanged and scales sV by 2^a exactly. With
    per-row B^T scales, row i of B^T times 2^k_i leaves the codes unchanged and
    scales sV at tap (i, j) by 2^(k_i + k_j); with one B^T scale, B^T * 2^k
    scales every sV by 2^(2k)."""
    rng = np.random.default_rng([12, m])
    n, G = m + 2, 32
    x = rng.standard_normal((1, 64, 2 * m + 3, 2 * m + 2)).astype(np.float32)
    Bt = std_bt(m)
    for rows in (False, True):
        Bq, sB = oracle.quant_bt(Bt, rows)
        Vq, sV = oracle.stage1_int(m, x, 1, G, Bq, sB)
        Vq2, sV2 = oracle.stage1_int(m, x * np.float32(8.0), 1, G, Bq, sB)
        assert np.array_equal(Vq, Vq2) and np.array_equal(sV2, sV * np.float32(8.0))
    k = rng.integers(-3, 4, size=n)
    Bt2 = (Bt * np.exp2(k)[:, None]).astype(np.float32)
    Bq, sB = oracle.quant_bt(Bt, True)
    Bq2, sB2 = oracle.quant_bt(Bt2, True)
    assert np.array_equal(Bq, Bq2) and np.array_equal(sB2, sB * np.exp2(k).astype(np.float32))
    Vq, sV = oracle.stage1_int(m, x, 1, G, Bq, sB)
    Vq2, sV2 = oracle.stage1_int(m, x, 1, G, Bq2, sB2)
    tapk = (k[:, None] + k[None, :]).reshape(-1)
    assert np.array_equal(Vq, Vq2)
    assert np.array_equal(sV2, sV * np.exp2(tapk).astype(np.float32)[:, None, None])
    Bq, sB = oracle.quant_bt(Bt, False)
    Bq2, sB2 = oracle.quant_bt(Bt * np.float32(4.0), False)
    Vq2, sV2 = oracle.stage1_int(m, x, 1, G, Bq2, sB2)
    Vq, sV = oracle.stage1_int(m, x, 1, G, Bq, sB)
    assert np.array_equal(Vq, Vq2) and np.array_equal(sV2, sV * np.float32(16.0))


@pytest.mark.parametrize("m,pad", [(4, 1), (6, 0), (6, 2)])
def test_patch_scale_covers_exactly_the_overlapping_tiles(m, pad):
    """A spike of 1000 at pixel (h0, w0) of one channel raises the patch scale
    to 1000/127 for exactly the tiles whose n x n input window (rows
    ty*m - pad ... ty*m - pad + n - 1, columns likewise) contains the pixel,
    and only for that channel's group."""
    rng = np.random.default_rng([13, m, pad])
    N, Cin, H, W, G = 1, 48, 3 * m + 1, 2 * m + 3, 16
    x = rng.uniform(-1, 1, size=(N, Cin, H, W)).astype(np.float32)
    h0, w0, c0 = m + 1, m, 21
    x[0, c0, h0, w0] = 1000.0
    Bq, sB = oracle.quant_bt(std_bt(m), False)
    _, _, _, sx = oracle.stage1_int(m, x, pad, G, Bq, sB, keep=True)
    tH, tW, T = oracle.tiles(m, N, H, W, pad)
    for t in range(T):
        ty, tx = t // tW, t % tW
        inside = (ty * m - pad <= h0 < ty * m - pad + m + 2) and (tx * m - pad <= w0 < tx * m - pad + m + 2)
        for g in range(Cin // G):
            hit = inside and g == c0 // G
            if hit:
                assert sx[t, g] == np.float32(1000.0) / np.float32(127.0)
            else:
                assert sx[t, g] <= np.float32(1.0) / np.float32(127.0)


@pytest.mark.parametrize("m,rows", [(4, False), (4, True), (6, True)])
def test_literal_error_bound(m, rows):
    """Dequantized V against the exact transform of the unquantized input.
    With Bd = diag(sB) Bq, E = Bd - B^T (|E_ik| <= sB_i / 2), dd = sx * dq
    (|dd - d| <= sx / 2):
      Bd dd Bd^T - B^T d B = Bd (dd - d) Bd^T + E d Bd^T + B^T d E^T,
    so each tap is off by at most the sum of the three absolute bounds, plus
    half a V step (sV / 2) and fp32 rounding of the scale products."""
    rng = np.random.default_rng([14, m, rows])
    n, G, pad = m + 2, 16, 1
    N, Cin, H, W = 1, 32, 2 * m + 2, 2 * m + 1
    x = rng.standard_normal((N, Cin, H, W)).astype(np.float32)
    Bt = std_bt(m, "f64")
    Bq, sB = oracle.quant_bt(Bt, rows, prec="f64")
    Vq, sV, xq, sx = oracle.stage1_int(m, x, pad, G, Bq, sB, prec="f64", keep=True)
    tH, tW, T = oracle.tiles(m, N, H, W, pad)
    Bd = sB[:, None] * Bq.astype(np.float64)
    E = np.abs(Bd - Bt)
    xp = np.zeros((N, Cin, tH * m + 2, tW * m + 2))
    hh, ww = min(H, tH * m + 2 - pad), min(W, tW * m + 2 - pad)
    xp[:, :, pad:pad + hh, pad:pad + ww] = x[:, :, :hh, :ww]
    worst = 0.0
    for t in range(T):
        ty, tx = t // tW, t % tW
        for c in range(Cin):
            d = xp[0, c, ty * m:ty * m + n, tx * m:tx * m + n]
            exact = Bt @ d @ Bt.T
            got = (Vq[:, t, c].astype(np.float64) * sV[:, t, c // G]).reshape(n, n)
            s = sx[t, c // G]
            bound = (np.abs(Bd) @ np.full((n, n), s / 2) @ np.abs(Bd).T
                     + E @ np.abs(d) @ np.abs(Bd).T + np.abs(Bt) @ np.abs(d) @ E.T
                     + sV[:, t, c // G].reshape(n, n) / 2)
            bound = bound * (1 + 1e-12) + 1e-12
            assert np.all(np.abs(got - exact) <= bound)
            worst = max(worst, float(np.max(np.abs(got - exact) / bound)))
    assert worst > 0.05  # the bound is not vacuous


def test_literal_forward_composes_the_stages():
    """forward(in_quant=...) is stage1_int followed by the pinned stages 2
    and 3 on the same codes."""
    rng = np.random.default_rng(15)
    m, G, pad = 6, 16, 1
    x = rng.standard_normal((1, 32, 9, 10)).astype(np.float32)
    w = (rng.standard_normal((8, 32, 3, 3)) * 0.1).astype(np.float32)
    for iq in ("int_tensor", "int_row"):
        r = oracle.forward(m, x, w, pad, G, keep=True, in_quant=iq)
        Bq, sB = oracle.quant_bt(r["Bt"], iq == "int_row")
        Vq, sV = oracle.stage1_int(m, x, pad, G, Bq, sB)
        assert np.array_equal(Vq, r["Vq"]) and np.array_equal(sV, r["sV"])
        y, _, _ = oracle.stage3(m, oracle.stage2(Vq, sV, r["Uq"], r["sU"], G), 1, 9, 10, pad, r["At"])
        assert np.array_equal(y, r["y"])
