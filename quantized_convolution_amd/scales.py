"""Diagonal transform scales for the quantized Winograd layer (offline tools).

The method's free parameters are the diagonal scales S_B and S_G of the
transforms B^T = S_B V^-T and G = S_G V (S_A = (S_B S_G)^-1 follows; "What
carries the argument" on the review page). The pages learn them without data
by minimising a quantization-error objective on random inputs (Algorithm 1,
SQNR objective Eq. 17 on the review page; "data-free" in the title); they do
not print the resulting values. This module provides two generators, both
run on the host before a plan is created:

  equalizing_scales  closed form: scale each transform row to unit norm, so
                     the Winograd-domain output Y has the same spread on every
                     tap for i.i.d. inputs and weights (the cross-shaped range
                     one Y scale cannot hold is what makes standard scales
                     collapse; core claim, Fig. 3 caption). An empirical
                     variant fits per-tap RMS of Y on noise instead.
  learn_scales       gradient descent on log S_B, log S_G of the output SQNR
                     of a fake-quantized layer (same quantization points and
                     groups as the library) on synthetic noise, with a
                     straight-through estimator for rounding.

Neither is on the hot path; the library only consumes the scales.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

INF = float("inf")


def standard_points(m: int):
    return {4: [0.0, 1.0, -1.0, 2.0, -2.0, INF],
            6: [0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, INF]}[m]


def _vander(points, cols):
    """Homogeneous Vandermonde rows: finite p -> p^j; infinity -> e_{cols-1}."""
    V = np.zeros((len(points), cols))
    for i, p in enumerate(points):
        if math.isinf(p):
            V[i, cols - 1] = 1.0
        else:
            V[i] = [p ** j for j in range(cols)]
    return V


def matrices(m, points, s_b, s_g):
    """Bt [n][n], G [n][3], At [m][n] in float64 for given scales."""
    n = m + 2
    V = _vander(points, n)
    Vinv = np.linalg.inv(V)
    V3 = _vander(points, 3)
    Vm = _vander(points, m)
    s_b, s_g = np.asarray(s_b, float), np.asarray(s_g, float)
    Bt = s_b[:, None] * Vinv.T
    G = s_g[:, None] * V3
    At = Vm.T * (1.0 / (s_b * s_g))[None, :]
    return Bt, G, At


def equalizing_scales(m: int, points=None, method: str = "closed", samples: int = 20000,
                      seed: int = 0):
    """(s_B, s_G) as float32 lists.

    method="closed": s_B[i] = 1/|row i of V^-T|, s_G[i] = 1/|row i of V_nx3|:
    for i.i.d. zero-mean data the std of Y[i][j] is proportional to
    |row i of B^T| |row i of G| |row j of B^T| |row j of G|, which this makes
    equal on every tap.
    method="empirical": per-tap RMS of Y = (G g G^T) * (B^T d B) with S = I on
    N(0, 1) patches and kernels, a separable least-squares fit of log RMS
    (log a_ij = u_i + u_j), then s_B s_G = exp(-u) with S_G normalising the
    rows of V_nx3 as above."""
    points = list(standard_points(m) if points is None else points)
    n = m + 2
    V = _vander(points, n)
    V3 = _vander(points, 3)
    g_norm = np.linalg.norm(V3, axis=1)
    if method == "closed":
        b_norm = np.linalg.norm(np.linalg.inv(V).T, axis=1)
        s_b, s_g = 1.0 / b_norm, 1.0 / g_norm
    elif method == "empirical":
        rng = np.random.default_rng(seed)
        Bt, G, _ = matrices(m, points, np.ones(n), np.ones(n))
        d = rng.standard_normal((samples, n, n))
        g = rng.standard_normal((samples, 3, 3))
        Y = np.einsum("ik,skl,jl->sij", G, g, G) * np.einsum("ik,skl,jl->sij", Bt, d, Bt)
        rms = np.sqrt(np.mean(Y ** 2, axis=0))
        # least squares for log rms_ij = u_i + u_j
        A = np.zeros((n * n, n))
        for i in range(n):
            for j in range(n):
                A[i * n + j, i] += 1
                A[i * n + j, j] += 1
        u = np.linalg.lstsq(A, np.log(rms).reshape(-1), rcond=None)[0]
        c = np.exp(-u)
        s_g = 1.0 / g_norm
        s_b = c / s_g
    else:
        raise ValueError(method)
    return [float(np.float32(v)) for v in s_b], [float(np.float32(v)) for v in s_g]


# --------------------------------------------------------------- learning
def _fake_quant(v, dims, ste=True):
    """Symmetric absmax int8 fake quantization over `dims` (torch)."""
    import torch

    a = v.abs().amax(dim=dims, keepdim=True)
    s = torch.where(a > 0, a / 127.0, torch.ones_like(a))
    r = v / s
    q = torch.clamp(torch.round(r), -127, 127)
    if ste:
        q = r + (q - r).detach()
    return q * s


def _layer_forward(m, points, log_sb, log_sg, x, w, G, pad=1):
    """Fake-quantized Winograd layer in float64 torch: V and U quantized per
    (tap, group of G channels), Y per (tile, co) over all taps, as in the
    library; returns the cropped output."""
    import torch
    import torch.nn.functional as F

    n = m + 2
    V = torch.tensor(_vander(points, n), dtype=torch.float64)
    Vinv = torch.linalg.inv(V)
    V3 = torch.tensor(_vander(points, 3), dtype=torch.float64)
    Vm = torch.tensor(_vander(points, m), dtype=torch.float64)
    sb, sg = torch.exp(log_sb), torch.exp(log_sg)
    Bt = sb[:, None] * Vinv.T
    Gm = sg[:, None] * V3
    At = Vm.T * (1.0 / (sb * sg))[None, :]

    N, C, H, W = x.shape
    Co = w.shape[0]
    Ho, Wo = H + 2 * pad - 2, W + 2 * pad - 2
    tH, tW = -(-Ho // m), -(-Wo // m)
    xp = F.pad(x, (pad, tW * m + 2 - W - pad, pad, tH * m + 2 - H - pad))
    d = xp.unfold(2, n, m).unfold(3, n, m)                       # [N][C][tH][tW][n][n]
    Vt = torch.einsum("ik,nchwkl,jl->nchwij", Bt, d, Bt)        # [N][C][tH][tW][n][n]
    ng = C // G
    Vg = Vt.reshape(N, ng, G, tH, tW, n, n)
    Vq = _fake_quant(Vg, dims=(2,)).reshape(N, C, tH, tW, n, n)
    U = torch.einsum("ia,ocab,jb->ocij", Gm, w, Gm)              # [Co][C][n][n]
    Uq = _fake_quant(U.reshape(Co, ng, G, n, n), dims=(2,)).reshape(Co, C, n, n)
    M = torch.einsum("nchwij,ocij->nohwij", Vq, Uq)
    Yq = _fake_quant(M, dims=(4, 5))
    O = torch.einsum("ai,nohwij,bj->nohwab", At, Yq, At)          # [N][Co][tH][tW][m][m]
    O = O.permute(0, 1, 2, 4, 3, 5).reshape(N, Co, tH * m, tW * m)
    return O[:, :, :Ho, :Wo]


def learn_scales(m: int, points=None, group: int = 64, steps: int = 200, lr: float = 0.05,
                 layers=((2, 64, 20, 20, 32),), seed: int = 0, init: str = "equalizing",
                 x_dist: str = "normal"):
    """Data-free learned scales: Adam on (log s_B, log s_G) minimising the
    negative output SQNR (dB) of the fake-quantized layer against the exact
    (float64) convolution, on fresh synthetic noise every step. `layers` are
    (N, Cin, H, W, Cout). Returns (s_B, s_G) as float32 lists and the loss
    history."""
    import torch
    import torch.nn.functional as F

    points = list(standard_points(m) if points is None else points)
    n = m + 2
    if init == "equalizing":
        b0, g0 = equalizing_scales(m, points)
    elif init == "identity":
        b0, g0 = [1.0] * n, [1.0] * n
    else:
        raise ValueError(init)
    log_sb = torch.tensor(np.log(b0), dtype=torch.float64, requires_grad=True)
    log_sg = torch.tensor(np.log(g0), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([log_sb, log_sg], lr=lr)
    gen = torch.Generator().manual_seed(seed)
    hist = []
    for _ in range(steps):
        loss = 0.0
        for (N, C, H, W, Co) in layers:
            if x_dist == "student_t":  # t with 3 dof, unit variance
                z = torch.randn((N, C, H, W), generator=gen, dtype=torch.float64)
                chi = torch.randn((3, N, C, H, W), generator=gen, dtype=torch.float64).pow(2).sum(0)
                x = z / torch.sqrt(chi / 3.0) / math.sqrt(3.0)
            else:
                x = torch.randn((N, C, H, W), generator=gen, dtype=torch.float64)
            w = torch.randn((Co, C, 3, 3), generator=gen, dtype=torch.float64) / math.sqrt(9 * C)
            ref = F.conv2d(x, w, padding=1)
            out = _layer_forward(m, points, log_sb, log_sg, x, w, group)
            err = torch.sum((out - ref) ** 2)
            loss = loss - 10.0 * torch.log10(torch.sum(ref ** 2) / err)
        loss = loss / len(layers)
        opt.zero_grad()
        loss.backward()
        opt.step()
        hist.append(float(loss.detach()))
    s_b = [float(np.float32(v)) for v in torch.exp(log_sb).detach().numpy()]
    s_g = [float(np.float32(v)) for v in torch.exp(log_sg).detach().numpy()]
    return s_b, s_g, hist


def learn_scales_model(m: int, layers, k: int = 3, steps: int = 300, lr: float = 0.02, seed: int = 0,
                       init: str = "identity", noise: str = "gaussian", points=None):
    """One shared (s_B, s_G) for a model's layers, learned without data: at
    every step, k of the `layers` are drawn at random; each runs on fresh
    noise inputs (zero-mean, unit variance: "gaussian" or "uniform") with
    its own fixed weights; the loss is the mean over the k layers of the
    negative output SQNR (dB) of the fake-quantized layer against the exact
    convolution; Adam updates log s_B and log s_G, with straight-through
    rounding. `layers` are dicts with w ([Cout][Cin][3][3] array), G, N, H,
    W. Returns (s_B, s_G) as float32 lists and the loss history."""
    import torch
    import torch.nn.functional as F

    points = list(standard_points(m) if points is None else points)
    n = m + 2
    if init == "equalizing":
        b0, g0 = equalizing_scales(m, points)
    elif init == "identity":
        b0, g0 = [1.0] * n, [1.0] * n
    else:
        raise ValueError(init)
    log_sb = torch.tensor(np.log(b0), dtype=torch.float64, requires_grad=True)
    log_sg = torch.tensor(np.log(g0), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([log_sb, log_sg], lr=lr)
    gen = torch.Generator().manual_seed(seed)
    ws = [torch.as_tensor(np.asarray(L["w"], np.float64)) for L in layers]
    hist = []
    for _ in range(steps):
        pick = torch.randperm(len(layers), generator=gen)[:k].tolist()
        loss = 0.0
        for i in pick:
            L, w = layers[i], ws[i]
            shape = (L["N"], w.shape[1], L["H"], L["W"])
            if noise == "gaussian":
                x = torch.randn(shape, generator=gen, dtype=torch.float64)
            elif noise == "uniform":
                x = (torch.rand(shape, generator=gen, dtype=torch.float64) * 2.0 - 1.0) * math.sqrt(3.0)
            else:
                raise ValueError(noise)
            ref = F.conv2d(x, w, padding=1)
            out = _layer_forward(m, points, log_sb, log_sg, x, w, L["G"])
            err = torch.sum((out - ref) ** 2)
            loss = loss - 10.0 * torch.log10(torch.sum(ref ** 2) / err)
        loss = loss / len(pick)
        opt.zero_grad()
        loss.backward()
        opt.step()
        hist.append(float(loss.detach()))
    s_b = [float(np.float32(v)) for v in torch.exp(log_sb).detach().numpy()]
    s_g = [float(np.float32(v)) for v in torch.exp(log_sg).detach().numpy()]
    return s_b, s_g, hist


# ------------------------------------------------------------ recorded sets
LEARNED_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data", "learned_scales.json")


def recorded_learned_scales(m: int):
    """(s_B, s_G) learned for F(m,3) by make_learned_scales.py, or None."""
    try:
        with open(LEARNED_FILE) as f:
            rec = json.load(f)
    except OSError:
        return None
    e = rec.get(f"F({m},3)")
    if e is None:
        return None
    return [float(v) for v in e["s_B"]], [float(v) for v in e["s_G"]]
