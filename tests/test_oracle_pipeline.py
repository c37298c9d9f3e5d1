"""Pins for the oracle's convolution and quantized pipeline (oracle/*.c).

Each test ties the oracle to something other than itself: a library routine
for the exact cases (torch conv2d in fp64), closed forms, the scale identity
S_A S_B S_G = I, power-of-two metamorphic relations, hand-computed quantizer
vectors, an independently written Kronecker-product formulation on tiny
inputs, and an a-posteriori error bound against the unquantized Winograd.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import transforms as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def rand_layer(seed, N, Cin, Cout, H, W):
    r = np.random.default_rng(seed)
    x = r.standard_normal((N, Cin, H, W)).astype(np.float32)
    w = (r.standard_normal((Cout, Cin, 3, 3)) * 0.3).astype(np.float32)
    return x, w


def pert_scales(seed, n):
    r = np.random.default_rng(seed)
    return (np.exp(r.uniform(-.5, .5, n)).astype(np.float32),
            np.exp(r.uniform(-.5, .5, n)).astype(np.float32))


# ------------------------------------------------------------ direct conv
@pytest.mark.parametrize("shape,pad", [((2, 3, 9, 7, 4), 1), ((1, 5, 6, 11, 2), 0),
                                       ((1, 2, 1, 1, 3), 1), ((1, 1, 4, 5, 1), 2)])
def test_direct_conv_matches_torch_fp64(shape, pad):
    N, Cin, H, W, Cout = shape
    x, w = rand_layer(1, N, Cin, Cout, H, W)
    ref = torch.nn.functional.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                                     padding=pad).numpy()
    y = oracle.direct_conv_f64(x, w, pad)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_direct_conv_closed_form_ones():
    # all-ones input and weights: each output counts the in-image taps times Cin
    x = np.ones((1, 4, 5, 6), np.float32)
    w = np.ones((2, 4, 3, 3), np.float32)
    y = oracle.direct_conv_f64(x, w, 1)
    rows = np.array([2, 3, 3, 3, 2])[:, None]
    cols = np.array([2, 3, 3, 3, 3, 2])[None, :]
    assert np.array_equal(y[0, 0], 4 * rows * cols)


# ------------------------------------------- unquantized Winograd (fp64)
SHAPES = [(1, 1, 1, 1, 1), (1, 2, 3, 3, 2), (2, 3, 7, 5, 2), (1, 2, 13, 14, 3),
          (1, 3, 8, 9, 1), (2, 2, 6, 6, 2), (1, 1, 2, 11, 1)]


@pytest.mark.parametrize("m", [4, 6])
@pytest.mark.parametrize("pad", [0, 1, 2])
@pytest.mark.parametrize("scales", ["identity", "perturbed"])
def test_unquantized_winograd_equals_direct(m, pad, scales):
    n = m + 2
    sb, sg = (np.ones(n, np.float32),) * 2 if scales == "identity" else pert_scales(m + pad, n)
    Bt, Gm, At = T.transforms_f64(m, T.standard_points(m), sb, sg)
    for k, (N, Cin, H, W, Cout) in enumerate(SHAPES):
        if H + 2 * pad - 2 < 1 or W + 2 * pad - 2 < 1:
            continue
        x, w = rand_layer(k, N, Cin, Cout, H, W)
        ya = oracle.direct_conv_f64(x, w, pad)
        yb = oracle.winograd_f64(m, x, w, pad, Bt, Gm, At)
        assert np.max(np.abs(ya - yb)) <= 1e-9 * rms(ya)


# ------------------------------------------------------ quantizer vectors
def _stage3_single(vals, m=6):
    """Run the Y quantizer on one (tile, co) holding the given n*n values."""
    n = m + 2
    M = np.zeros((n * n, 1, 1), np.float32)
    M[:, 0, 0] = vals
    At = np.zeros((m, n), np.float32)
    y, Yq, sY = oracle.stage3(m, M, 1, m, m, 1, At)
    return Yq[0, 0], sY[0, 0]


def test_quantizer_hand_vectors():
    v = np.zeros(64, np.float32)
    v[:8] = [127, 2.5, 3.5, -2.5, 0.5, 1.5, -127, -0.49]
    q, s = _stage3_single(v)
    # absmax 127 -> 127/a = 1 exactly, codes are rint (ties to even)
    assert s == np.float32(1.0)
    assert list(q[:8]) == [127, 2, 4, -2, 0, 2, -127, 0]
    assert not q[8:].any()


def test_quantizer_scale_and_extremes():
    v = np.zeros(64, np.float32)
    v[5], v[9] = np.float32(-3.0), np.float32(1.5)
    q, s = _stage3_single(v)
    assert s == np.float32(3.0) / np.float32(127.0)
    assert q[5] == -127 and q[9] == 64          # 1.5 * (127/3) = 63.5 -> tie -> 64
    q, s = _stage3_single(np.zeros(64, np.float32))
    assert s == 0 and not q.any()               # all-zero group
    q, s = _stage3_single(np.full(64, np.float32(7.25)))
    assert (q == 127).all() and s == np.float32(7.25) / np.float32(127.0)


def test_quantizer_single_element_groups():
    # G = 1: every value is its own group -> code +-127 (or 0), scale |v|/127
    x, w = rand_layer(3, 1, 2, 1, 5, 5)
    Bt, Gm, At = T.transforms_f32(4, T.standard_points(4), np.ones(6), np.ones(6))
    Vq, sV = oracle.stage1(4, x, 1, 1, Bt)
    nz = sV[..., 0] != 0
    assert (np.abs(Vq[..., 0][nz]) == 127).all() and (Vq[..., 0][~nz] == 0).all()


# --------------------------------------------------- metamorphic relations
@pytest.mark.parametrize("m", [4, 6])
def test_power_of_two_scales_keep_codes(m):
    n = m + 2
    x, w = rand_layer(7, 1, 8, 4, 2 * m + 3, 3 * m + 1)
    base = oracle.forward(m, x, w, 1, 4, keep=True)
    r = np.random.default_rng(m)
    kb, kg = r.integers(-3, 4, n), r.integers(-3, 4, n)
    sb, sg = np.float32(2.0) ** kb, np.float32(2.0) ** kg
    out = oracle.forward(m, x, w, 1, 4, s_b=sb, s_g=sg, keep=True)
    assert np.array_equal(out["Vq"], base["Vq"]) and np.array_equal(out["Uq"], base["Uq"])
    tap_b = (2.0 ** (kb[:, None] + kb[None, :])).reshape(-1)
    tap_g = (2.0 ** (kg[:, None] + kg[None, :])).reshape(-1)
    assert np.array_equal(out["sV"], (base["sV"] * tap_b[:, None, None]).astype(np.float32))
    assert np.array_equal(out["sU"], (base["sU"] * tap_g[:, None, None]).astype(np.float32))


@pytest.mark.parametrize("m", [4, 6])
def test_uniform_power_of_two_scale_is_bit_identical(m):
    n = m + 2
    x, w = rand_layer(8, 2, 8, 4, 2 * m + 1, 2 * m + 5)
    base = oracle.forward(m, x, w, 1, 8)
    out = oracle.forward(m, x, w, 1, 8, s_b=np.full(n, 4.0, np.float32),
                         s_g=np.full(n, 0.125, np.float32))
    assert np.array_equal(base, out)


@pytest.mark.parametrize("m", [4, 6])
def test_point_permutation_permutes_taps(m):
    n = m + 2
    x, w = rand_layer(9, 1, 4, 3, 2 * m + 2, 2 * m - 1)
    pts = np.array(T.standard_points(m))
    sb, sg = pert_scales(9, n)
    perm = np.random.default_rng(m).permutation(n)
    a = oracle.forward(m, x, w, 1, 4, points=list(pts), s_b=sb, s_g=sg, keep=True)
    b = oracle.forward(m, x, w, 1, 4, points=list(pts[perm]), s_b=sb[perm], s_g=sg[perm],
                       keep=True)
    tp = (perm[:, None] * n + perm[None, :]).reshape(-1)  # new tap -> old tap
    assert np.array_equal(b["Vq"], a["Vq"][tp]) and np.array_equal(b["sV"], a["sV"][tp])
    assert np.array_equal(b["Uq"], a["Uq"][tp]) and np.array_equal(b["M"], a["M"][tp])
    assert np.array_equal(b["Yq"], a["Yq"][..., tp]) and np.array_equal(b["sY"], a["sY"])
    np.testing.assert_allclose(b["y"], a["y"], rtol=0, atol=1e-5 * rms(a["y"]))


# ------------------------------------------------ brute force, Kronecker
def _q(v):
    a = np.max(np.abs(v))
    if a == 0:
        return np.zeros(v.shape, np.int8), 0.0
    inv = 127.0 / a
    return np.clip(np.rint(v * inv), -127, 127).astype(np.int8), a / 127.0


def kron_pipeline(m, x, w, pad, G, Bt, Gm, At, y_group="tile"):
    """Independent formulation on whole tiles: vec(B d B^T) = (B kron B) vec(d)."""
    n = m + 2
    N, Cin, H, W = x.shape
    Cout = w.shape[0]
    Ho, Wo = H + 2 * pad - 2, W + 2 * pad - 2
    tH, tW = -(-Ho // m), -(-Wo // m)
    KB, KG, KA = np.kron(Bt, Bt), np.kron(Gm, Gm), np.kron(At, At)
    xp = np.zeros((N, Cin, tH * m + 2, tW * m + 2))
    xp[:, :, pad:pad + H, pad:pad + W] = x
    ng = Cin // G
    # weights: U[co, ci, tap]
    U = np.einsum("tk,ock->oct", KG, w.reshape(Cout, Cin, 9).astype(np.float64))
    Uq = np.zeros((n * n, Cout, Cin), np.int8)
    sU = np.zeros((n * n, Cout, ng))
    for co in range(Cout):
        for tap in range(n * n):
            for g in range(ng):
                Uq[tap, co, g * G:(g + 1) * G], sU[tap, co, g] = _q(U[co, g * G:(g + 1) * G, tap])
    T_ = N * tH * tW
    Vq = np.zeros((n * n, T_, Cin), np.int8)
    sV = np.zeros((n * n, T_, ng))
    Yq = np.zeros((T_, Cout, n * n), np.int8)
    sY = np.zeros((T_, Cout)) if y_group == "tile" else np.zeros((T_, Cout, n))
    y = np.zeros((N, Cout, tH * m, tW * m))
    t = 0
    for img in range(N):
        for ty in range(tH):
            for tx in range(tW):
                d = xp[img, :, ty * m:ty * m + n, tx * m:tx * m + n].reshape(Cin, n * n)
                V = d @ KB.T                                   # [ci, tap]
                for tap in range(n * n):
                    for g in range(ng):
                        Vq[tap, t, g * G:(g + 1) * G], sV[tap, t, g] = _q(V[g * G:(g + 1) * G, tap])
                for co in range(Cout):
                    Mv = np.zeros(n * n)
                    for tap in range(n * n):
                        for g in range(ng):
                            sl = slice(g * G, (g + 1) * G)
                            P = int(np.dot(Vq[tap, t, sl].astype(np.int64), Uq[tap, co, sl].astype(np.int64)))
                            Mv[tap] += sV[tap, t, g] * sU[tap, co, g] * P
                    if y_group == "tile":
                        Yq[t, co], sY[t, co] = _q(Mv)
                        o = (KA @ Yq[t, co].astype(np.float64)) * sY[t, co]
                    else:  # one scale per row of taps, applied before the transform
                        Yd = np.zeros(n * n)
                        for i in range(n):
                            Yq[t, co, i * n:(i + 1) * n], sY[t, co, i] = _q(Mv[i * n:(i + 1) * n])
                            Yd[i * n:(i + 1) * n] = sY[t, co, i] * Yq[t, co, i * n:(i + 1) * n]
                        o = KA @ Yd
                    y[img, co, ty * m:(ty + 1) * m, tx * m:(tx + 1) * m] = o.reshape(m, m)
                t += 1
    return dict(Uq=Uq, sU=sU, Vq=Vq, sV=sV, Yq=Yq, sY=sY, y=y[:, :, :Ho, :Wo])


@pytest.mark.parametrize("y_group", ["tile", "row"])
@pytest.mark.parametrize("m", [4, 6])
def test_brute_force_kronecker_tiny(m, y_group):
    n = m + 2
    r = np.random.default_rng(40 + m)
    cases = 0
    for C in (1, 2, 4):
        for G in sorted({1, C // 2 or 1, C}):
            for _ in range(4):
                pad = int(r.integers(0, 2))
                H = int(r.integers(3 - 2 * pad, 2 * m + 3))
                W = int(r.integers(3 - 2 * pad, 2 * m + 3))
                x, w = rand_layer(int(r.integers(1 << 30)), 1, C, C, H, W)
                sb, sg = pert_scales(int(r.integers(1 << 30)), n)
                Bt, Gm, At = T.transforms_f64(m, T.standard_points(m), sb, sg)
                ref = kron_pipeline(m, x, w, pad, G, Bt, Gm, At, y_group)
                got = oracle.forward(m, x, w, pad, G, s_b=sb, s_g=sg, prec="f64", keep=True,
                                     y_group=y_group)
                for k in ("Uq", "Vq", "Yq"):
                    assert np.array_equal(got[k], ref[k]), (k, C, G, H, W, pad)
                for k in ("sU", "sV", "sY"):
                    np.testing.assert_allclose(got[k], ref[k], rtol=1e-9, atol=0)
                np.testing.assert_allclose(got["y"], ref["y"], rtol=1e-9,
                                           atol=1e-12 * max(rms(ref["y"]), 1e-300))
                cases += 1
    assert cases >= 20


# ------------------------------------------------- a-posteriori error bound
@pytest.mark.parametrize("m,G,scales", [(4, 8, "identity"), (6, 8, "perturbed"),
                                        (6, 4, "identity"), (4, 16, "perturbed")])
def test_error_bound_against_unquantized(m, G, scales):
    """|O-C - O-B| <= sum_ij |At_ai||At_bj| (E_M[i][j] + sY/2) + slop, where
    E_M = sum_c (|V~| sU/2 + |U~| sV/2 + sV sU/4) bounds the Hadamard error from
    rounding V and U to codes (V~ = sV Vq, U~ = sU Uq) and sY/2 the Y rounding."""
    n = m + 2
    N, Cin, Cout, H, W = 1, 16, 4, 2 * m + 3, 3 * m + 1
    x, w = rand_layer(20 + m + G, N, Cin, Cout, H, W)
    sb, sg = (np.ones(n, np.float32),) * 2 if scales == "identity" else pert_scales(m, n)
    q = oracle.forward(m, x, w, 1, G, s_b=sb, s_g=sg, keep=True)
    B64, G64, A64 = T.transforms_f64(m, T.standard_points(m), sb, sg)
    yb = oracle.winograd_f64(m, x, w, 1, B64, G64, A64)
    ng = Cin // G
    Vd = q["Vq"].astype(np.float64) * np.repeat(q["sV"].astype(np.float64), G, axis=2)
    Ud = q["Uq"].astype(np.float64) * np.repeat(q["sU"].astype(np.float64), G, axis=2)
    sVr = np.repeat(q["sV"].astype(np.float64), G, axis=2)      # [tap][t][ci]
    sUr = np.repeat(q["sU"].astype(np.float64), G, axis=2)      # [tap][co][ci]
    # E_M[tap][t][co]
    EM = (np.einsum("ptc,poc->pto", np.abs(Vd), sUr / 2) + np.einsum("ptc,poc->pto", sVr / 2, np.abs(Ud))
          + np.einsum("ptc,poc->pto", sVr, sUr) / 4)
    mag = np.einsum("ptc,poc->pto", np.abs(Vd), np.abs(Ud))     # size of the Hadamard terms
    # fp32 rounding in V itself, relative to sum |Bt||d||Bt|
    xa = np.abs(x.astype(np.float64))
    Babs = np.abs(B64)
    Ho, Wo = H + 2 - 2, W + 2 - 2
    tH, tW = -(-Ho // m), -(-Wo // m)
    xp = np.zeros((N, Cin, tH * m + 2, tW * m + 2))
    xp[:, :, 1:1 + H, 1:1 + W] = xa
    vmag = np.zeros_like(Vd)
    t = 0
    for ty in range(tH):
        for tx in range(tW):
            d = xp[0, :, ty * m:ty * m + n, tx * m:tx * m + n]
            vmag[:, t, :] = np.einsum("ik,ckl,jl->cij", Babs, d, Babs).reshape(Cin, n * n).T
            t += 1
    EM += 1e-5 * (mag + np.einsum("ptc,poc->pto", vmag, np.abs(Ud)))
    sY = q["sY"].astype(np.float64)                               # [t][co]
    Aabs = np.abs(A64)
    KA = np.kron(Aabs, Aabs)                                      # [(a,b)][(i,j)]
    bound = np.einsum("ap,pto->toa", KA, EM) + np.einsum("ap->a", KA)[None, None, :] * sY[..., None] * (0.5 + 1e-5 * 127)
    bound = bound.reshape(tH, tW, Cout, m, m).transpose(2, 0, 3, 1, 4).reshape(Cout, tH * m, tW * m)
    err = np.abs(q["y"][0].astype(np.float64) - yb[0])
    assert (err <= bound[:, :Ho, :Wo]).all()
    assert np.max(err / bound[:, :Ho, :Wo]) > 1e-3   # the bound is not vacuous


# ---------------------------------------------------------- int32 partials
def test_stage2_i32_matches_integer_matmul():
    r = np.random.default_rng(2)
    n2, T_, Cin, Cout, G = 9, 37, 96, 20, 32
    Vq = r.integers(-127, 128, (n2, T_, Cin), dtype=np.int8)
    Uq = r.integers(-127, 128, (n2, Cout, Cin), dtype=np.int8)
    P = oracle.stage2_i32(Vq, Uq, G)
    for g in range(Cin // G):
        sl = slice(g * G, (g + 1) * G)
        ref = np.matmul(Vq[:, :, sl].astype(np.int64), Uq[:, :, sl].astype(np.int64).transpose(0, 2, 1))
        assert np.array_equal(P[:, g], ref)


def test_stage2_single_group_is_one_rounding():
    # one group: M = fma(sV sU, P, 0) = fl32(fl32(sV sU) * P)
    r = np.random.default_rng(4)
    Vq = r.integers(-127, 128, (4, 5, 16), dtype=np.int8)
    Uq = r.integers(-127, 128, (4, 3, 16), dtype=np.int8)
    sV = r.uniform(0.01, 1, (4, 5, 1)).astype(np.float32)
    sU = r.uniform(0.01, 1, (4, 3, 1)).astype(np.float32)
    M = oracle.stage2(Vq, sV, Uq, sU, 16)
    P = np.einsum("ptc,poc->pto", Vq.astype(np.int64), Uq.astype(np.int64)).astype(np.float64)
    s = (sV * sU.transpose(0, 2, 1)).astype(np.float32).astype(np.float64)
    assert np.array_equal(M, (s * P).astype(np.float32))


# ------------------------------------------------- threads do not matter
def test_thread_count_does_not_change_bits():
    code = ("import numpy as np, oracle, sys;"
            "r=np.random.default_rng(5);"
            "x=r.standard_normal((2,16,17,19)).astype(np.float32);"
            "w=r.standard_normal((8,16,3,3)).astype(np.float32);"
            "y=oracle.forward(6,x,w,1,8);"
            "sys.stdout.write(y.tobytes().hex()[:0]+str(hash(y.tobytes())))")
    outs = []
    for th in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=th, PYTHONHASHSEED="0", PYTHONPATH=ROOT)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT,
                                   capture_output=True, text=True, check=True).stdout)
    assert outs[0] == outs[1]


# ------------------------------------------------------- the pages' claim
def _eq_scales(m):
    with open(os.path.join(ROOT, "tests", "golden", "equalized_scales.json")) as f:
        d = json.load(f)[f"F({m},3)"]
    return np.array(d["s_B"], np.float32), np.array(d["s_G"], np.float32)


def test_standard_scales_collapse_and_equalized_recover():
    """Qualitative (the pages print no SQNR values): with one Y scale per
    (tile, co) the standard scales collapse F(6,3), scales that even out the
    taps recover it, and F(4,3) is better than F(6,3)."""
    r = np.random.default_rng(12)
    x = np.maximum(r.standard_normal((2, 64, 20, 20)), 0).astype(np.float32)
    w = (r.standard_normal((64, 64, 3, 3)) * np.sqrt(2 / (9 * 64))).astype(np.float32)
    ya = oracle.direct_conv_f64(x, w, 1)
    s = {}
    for m in (4, 6):
        s[m, "I"] = oracle.sqnr_db(ya, oracle.forward(m, x, w, 1, 64))
        sb, sg = _eq_scales(m)
        s[m, "eq"] = oracle.sqnr_db(ya, oracle.forward(m, x, w, 1, 64, s_b=sb, s_g=sg))
    assert s[6, "I"] < 0 < 10 < s[6, "eq"]
    assert s[4, "I"] < s[4, "eq"] - 10
    assert s[4, "eq"] > s[6, "eq"]


# ----------------------------------------------------------------- bf16
def test_bf16_helpers_match_torch():
    r = np.random.default_rng(6)
    v = (r.standard_normal(10000) * 10.0 ** r.integers(-5, 5, 10000)).astype(np.float32)
    bits = oracle.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = oracle.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ------------------------------------------------ sampled evaluation
@pytest.mark.parametrize("m,G", [(6, 16), (4, 32)])
def test_sampled_equals_full_pipeline(m, G):
    # the per-pair evaluation must reproduce the full stages bit for bit
    x, w = rand_layer(31, 2, 64, 24, 2 * m + 5, 3 * m - 1)
    sb, sg = pert_scales(31, m + 2)
    q = oracle.forward(m, x, w, 1, G, s_b=sb, s_g=sg, keep=True)
    T_ = q["M"].shape[1]
    r = np.random.default_rng(3)
    pairs = np.stack([r.integers(0, T_, 40), r.integers(0, 24, 40)], 1)
    Ms, Yq, sY, ys = oracle.sampled(m, q["Vq"], q["sV"], q["Uq"], q["sU"], q["At"], pairs)
    assert np.array_equal(Ms, q["M"][:, pairs[:, 0], pairs[:, 1]].T)
    assert np.array_equal(Yq, q["Yq"][pairs[:, 0], pairs[:, 1]])
    assert np.array_equal(sY, q["sY"][pairs[:, 0], pairs[:, 1]])
    N, _, H, W = x.shape
    Ho, Wo = H, W
    tH, tW = -(-Ho // m), -(-Wo // m)
    for s, (t, co) in enumerate(pairs):
        img, ty, tx = t // (tH * tW), t // tW % tH, t % tW
        blk = q["y"][img, co, ty * m:(ty + 1) * m, tx * m:(tx + 1) * m]
        assert np.array_equal(ys[s][:blk.shape[0], :blk.shape[1]], blk)
