"""Pins for the oracle's group-wise W8A8 direct convolution (the non-Winograd
baseline of the pages' speed comparison: group-quantized direct kernels,
summary page Fig. 6 caption).

Each pin fixes the answer independently of the oracle's own code: exact
integer arithmetic when the inputs are already code-valued, an independent
numpy re-derivation on tiny inputs, an exact power-of-two scaling identity,
and an a-posteriori error bound against the fp64 direct convolution.
"""
import numpy as np
import pytest

import oracle


def code_valued(shape_outer, G, Cin, rng, axis_len_last=True):
    """Integers in [-127, 127] whose every group of G along the channel axis
    holds +-127 at least once (so absmax = 127, scale = 1, codes = values)."""
    v = rng.integers(-127, 128, size=shape_outer + (Cin,)).astype(np.float32)
    ng = Cin // G
    idx = rng.integers(0, G, size=shape_outer + (ng,))
    sign = np.where(rng.random(shape_outer + (ng,)) < 0.5, -127.0, 127.0).astype(np.float32)
    for g in range(ng):
        np.put_along_axis(v[..., g * G:(g + 1) * G], idx[..., g:g + 1], sign[..., g:g + 1], axis=-1)
    return v


@pytest.mark.parametrize("pad", [0, 1, 2])
@pytest.mark.parametrize("G", [16, 32])
def test_w8a8_exact_on_code_valued_inputs(pad, G):
    rng = np.random.default_rng([7, pad, G])
    N, Cin, Cout, H, W = 2, 32, 5, 7, 6
    x_nhwc = code_valued((N, H, W), G, Cin, rng)
    x = np.ascontiguousarray(x_nhwc.transpose(0, 3, 1, 2))
    w_tap = code_valued((Cout, 9), G, Cin, rng)            # [Cout][tap][Cin]
    w = np.ascontiguousarray(w_tap.transpose(0, 2, 1).reshape(Cout, Cin, 3, 3))
    r = oracle.direct_w8a8(x, w, pad, G, keep=True)
    assert np.all(r["sx"] == 1.0) and np.all(r["sw"] == 1.0)
    assert np.array_equal(r["xq"].astype(np.float32), x_nhwc)
    # every partial sum is an integer below 2^24: the fp32 chain is exact
    ref = oracle.direct_conv_f64(x, w, pad)
    assert np.array_equal(r["y"].astype(np.float64), ref)


def _quant_np(v, axis_groups):
    """Absmax quantizer in float64 along the last axis (groups already split)."""
    a = np.max(np.abs(v), axis=-1, keepdims=True)
    safe = np.where(a == 0, 1.0, a)
    q = np.clip(np.rint(v * (127.0 / safe)), -127, 127)
    q = np.where(a == 0, 0, q).astype(np.int8)
    s = np.where(a == 0, 0.0, a / 127.0)[..., 0]
    return q, s


@pytest.mark.parametrize("pad", [0, 1])
def test_w8a8_matches_numpy_rederivation(pad):
    """Indices, shifts, padding and grouping: the fp64 build against a
    separately written numpy formulation (same quantizer rule, different
    loop structure and summation order)."""
    rng = np.random.default_rng([8, pad])
    N, Cin, Cout, H, W, G = 1, 24, 3, 5, 6, 8
    x = rng.standard_normal((N, Cin, H, W)).astype(np.float32)
    w = (0.3 * rng.standard_normal((Cout, Cin, 3, 3))).astype(np.float32)
    r = oracle.direct_w8a8(x, w, pad, G, prec="f64", keep=True)
    ng = Cin // G
    xg = x.astype(np.float64).transpose(0, 2, 3, 1).reshape(N, H, W, ng, G)
    xq, sx = _quant_np(xg, None)
    wg = w.astype(np.float64).reshape(Cout, ng, G, 9).transpose(3, 0, 1, 2)  # [tap][co][g][c]
    wq, sw = _quant_np(wg, None)
    assert np.array_equal(r["xq"], xq.reshape(N, H, W, Cin))
    assert np.array_equal(r["wq"], wq.reshape(9, Cout, Cin))
    Ho, Wo = H + 2 * pad - 2, W + 2 * pad - 2
    y = np.zeros((N, Cout, Ho, Wo))
    xpad = np.zeros((N, H + 2 * pad, W + 2 * pad, ng, G))
    spad = np.zeros((N, H + 2 * pad, W + 2 * pad, ng))
    xpad[:, pad:pad + H, pad:pad + W] = xq
    spad[:, pad:pad + H, pad:pad + W] = sx
    for kh in range(3):
        for kw in range(3):
            xs = xpad[:, kh:kh + Ho, kw:kw + Wo]          # [N][Ho][Wo][g][c]
            ss = spad[:, kh:kh + Ho, kw:kw + Wo]          # [N][Ho][Wo][g]
            P = np.einsum("nhwgc,ogc->nohwg", xs, wq[kh * 3 + kw].astype(np.float64))
            y += np.einsum("nohwg,nhwg,og->nohw", P, ss, sw[kh * 3 + kw])
    np.testing.assert_allclose(r["y"], y, rtol=1e-12, atol=1e-12 * np.max(np.abs(y)))


def test_w8a8_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 32, 6, 7)).astype(np.float32)
    w = (0.1 * rng.standard_normal((4, 32, 3, 3))).astype(np.float32)
    a = oracle.direct_w8a8(x, w, 1, 16, keep=True)
    b = oracle.direct_w8a8(x * np.float32(8.0), w, 1, 16, keep=True)
    assert np.array_equal(a["xq"], b["xq"])
    assert np.array_equal(a["sx"] * np.float32(8.0), b["sx"])
    assert np.array_equal(a["y"] * np.float32(8.0), b["y"])


@pytest.mark.parametrize("G", [16, 64])
def test_w8a8_error_bound_against_fp64(G):
    """|y_q - y| <= sum over taps and channels of |x| sw/2 + |w| sx/2 +
    sx sw/4 (each operand off by at most half a step), plus fp32 slack."""
    rng = np.random.default_rng([10, G])
    N, Cin, Cout, H, W, pad = 1, 64, 6, 6, 5, 1
    x = rng.standard_normal((N, Cin, H, W)).astype(np.float32)
    w = (0.2 * rng.standard_normal((Cout, Cin, 3, 3))).astype(np.float32)
    r = oracle.direct_w8a8(x, w, pad, G, keep=True)
    ref = oracle.direct_conv_f64(x, w, pad)
    ng = Cin // G
    Ho, Wo = H + 2 * pad - 2, W + 2 * pad - 2
    sx = r["sx"].astype(np.float64)                       # [N][H][W][g]
    sw = r["sw"].astype(np.float64)                       # [tap][co][g]
    xa = np.abs(x.astype(np.float64))
    wa = np.abs(w.astype(np.float64))
    bound = np.zeros((N, Cout, Ho, Wo))
    mag = np.zeros((N, Cout, Ho, Wo))
    for kh in range(3):
        for kw in range(3):
            tap = kh * 3 + kw
            for ho in range(Ho):
                for wo in range(Wo):
                    h, wc = ho + kh - pad, wo + kw - pad
                    if not (0 <= h < H and 0 <= wc < W):
                        continue
                    for g in range(ng):
                        cs = slice(g * G, (g + 1) * G)
                        xs = xa[:, cs, h, wc]                     # [N][G]
                        ws = wa[:, cs, kh, kw]                    # [co][G]
                        e = (xs.sum(1)[:, None] * sw[tap, :, g][None, :] / 2
                             + ws.sum(1)[None, :] * sx[:, h, wc, g][:, None] / 2
                             + G * sx[:, h, wc, g][:, None] * sw[tap, :, g][None, :] / 4)
                        bound[:, :, ho, wo] += e
                        mag[:, :, ho, wo] += (xs @ ws.T)
    err = np.abs(r["y"].astype(np.float64) - ref)
    assert np.all(err <= bound + 1e-5 * mag + 1e-30)
    assert np.max(err / (bound + 1e-30)) > 1e-3      # the bound is not vacuous
