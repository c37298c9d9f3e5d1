"""Seeded synthetic layers for the quantized Winograd convolution.

This module only draws random inputs; it holds none of the method's
arithmetic, so the CPU oracle and the HIP library can both be fed from it.

The shapes stand in for the workloads the paper evaluates (ResNet-18/34 3x3
layers on ImageNet, Stable-Diffusion-v1.5 UNet 3x3 layers; experimental-setup
section of the AI summary page, referee summary of the review page). Their
datasets and weights are not used: activations and weights are drawn from
the distributions below.

Seeds: numpy default_rng([cfg_id, layer_idx, stream]) with stream
0 = x, 1 = w, 2 = s_B, 3 = s_G, 4 = outlier-channel choice.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

INF = float("inf")

STANDARD_POINTS = {
    4: (0.0, 1.0, -1.0, 2.0, -2.0, INF),
    6: (0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, INF),
}


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    cfg_id: int
    layer_idx: int
    m: int
    N: int
    Cin: int
    Cout: int
    H: int
    W: int
    pad: int
    G: int
    x_dist: str          # normal | relu_normal | student_t | student_t_outliers
    w_std: float | None  # None = He-normal, std sqrt(2 / (9 Cin))
    scales: str          # identity | perturbed

    @property
    def n(self):
        return self.m + 2

    @property
    def Ho(self):
        return self.H + 2 * self.pad - 2

    @property
    def Wo(self):
        return self.W + 2 * self.pad - 2

    @property
    def tiles(self):
        return self.N * math.ceil(self.Ho / self.m) * math.ceil(self.Wo / self.m)

    def direct_ops(self) -> int:
        """Operations of the equivalent direct convolution (2 per MAC)."""
        return 2 * self.N * self.Cin * self.Cout * self.Ho * self.Wo * 9

    def replace(self, **kw) -> "Layer":
        return dataclasses.replace(self, **kw)


def _layers():
    L = []
    L.append(Layer("c1_f4_n1_c16_16x16_g16", 1, 0, 4, 1, 16, 16, 16, 16, 1, 16,
                   "normal", 0.1, "identity"))
    L.append(Layer("c2_f6_n32_c64_56x56_g64", 2, 0, 6, 32, 64, 64, 56, 56, 1, 64,
                   "relu_normal", None, "perturbed"))
    for i, (c, hw) in enumerate(((128, 28), (256, 14), (512, 7))):
        L.append(Layer(f"c3{'abc'[i]}_f6_n32_c{c}_{hw}x{hw}_g64", 3, i, 6, 32, c, c, hw, hw, 1,
                       64, "relu_normal", None, "perturbed"))
    for m in (4, 6):
        for sc in ("identity", "perturbed"):
            L.append(Layer(f"c4_f{m}_n2_c320_64x64_g64_{'std' if sc == 'identity' else 'pert'}",
                           4, 0, m, 2, 320, 320, 64, 64, 1, 64, "student_t", 0.02, sc))
    for i, (c, hw) in enumerate(((640, 32), (1280, 16))):
        for g in (32, 128):
            L.append(Layer(f"c5_f6_n8_c{c}_{hw}x{hw}_g{g}", 5, i, 6, 8, c, c, hw, hw, 1, g,
                           "student_t_outliers", 0.02, "perturbed"))
    return {l.name: l for l in L}


LAYERS = _layers()
BENCH_LAYER = "c2_f6_n32_c64_56x56_g64"


def rng(layer: Layer, stream: int) -> np.random.Generator:
    return np.random.default_rng([layer.cfg_id, layer.layer_idx, stream])


def make_x(layer: Layer) -> np.ndarray:
    r = rng(layer, 0)
    shape = (layer.N, layer.Cin, layer.H, layer.W)
    if layer.x_dist == "normal":
        x = r.standard_normal(shape)
    elif layer.x_dist == "relu_normal":
        x = np.maximum(r.standard_normal(shape), 0.0)
    elif layer.x_dist in ("student_t", "student_t_outliers"):
        x = r.standard_t(3, shape) / math.sqrt(3.0)
        if layer.x_dist == "student_t_outliers":
            k = max(1, round(0.01 * layer.Cin))
            ch = rng(layer, 4).choice(layer.Cin, size=k, replace=False)
            x[:, ch] *= 20.0
    else:
        raise ValueError(layer.x_dist)
    return np.ascontiguousarray(x, dtype=np.float32)


def make_w(layer: Layer) -> np.ndarray:
    r = rng(layer, 1)
    std = math.sqrt(2.0 / (9 * layer.Cin)) if layer.w_std is None else layer.w_std
    w = r.standard_normal((layer.Cout, layer.Cin, 3, 3)) * std
    return np.ascontiguousarray(w, dtype=np.float32)


def make_scales(layer: Layer):
    """(s_B, s_G) as fp32; 'perturbed' draws exp(U(-1/2, 1/2)) per entry."""
    n = layer.n
    if layer.scales == "identity":
        return np.ones(n, np.float32), np.ones(n, np.float32)
    sb = np.exp(rng(layer, 2).uniform(-0.5, 0.5, n)).astype(np.float32)
    sg = np.exp(rng(layer, 3).uniform(-0.5, 0.5, n)).astype(np.float32)
    return sb, sg


def make(layer: Layer) -> dict:
    sb, sg = make_scales(layer)
    return dict(x=make_x(layer), w=make_w(layer), s_b=sb, s_g=sg,
                points=np.array(STANDARD_POINTS[layer.m], np.float64))


def small(layer: Layer, N=1, H=None, W=None, Cin=None, Cout=None) -> Layer:
    """Same distributions and group size at a size the CPU oracle finishes in
    seconds; the default spatial size spans several tiles and a ragged tail."""
    H = H if H is not None else 2 * layer.m + 3
    W = W if W is not None else 3 * layer.m + 1
    Cin = Cin if Cin is not None else max(layer.G, min(layer.Cin, 2 * layer.G))
    Cout = Cout if Cout is not None else min(layer.Cout, 48)
    return layer.replace(name=layer.name + f"_small_n{N}_c{Cin}x{Cout}_{H}x{W}",
                         N=N, H=H, W=W, Cin=Cin, Cout=Cout)
