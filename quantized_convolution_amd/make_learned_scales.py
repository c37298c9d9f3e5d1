"""Writes data/learned_scales.json: one learned (S_B, S_G) per F(m,3), shared
by the benchmark layers of that m (offline; not on the hot path).

The procedure follows the pages' data-free scale learning (review page,
referee summary and major comment 4; summary page, "Approach"): the model's
weights stay fixed, the inputs are random noise, K layers are drawn per
iteration, and the one shared set of scales is updated to raise the layers'
output SQNR against full precision, with straight-through rounding. The pages
do not state K, the step count, the learning rate or the noise magnitude;
the values below are this tool's choice and are recorded in the file.

The "model" is the set of benchmark layers of each m with their seeded
weights (workloads.py), each cut to at most 256 input and 32 output channels
and a 14 x 14 input to keep the float64 fake-quantized layer cheap; the group
size stays the layer's own.

Run: python -m quantized_convolution_amd.make_learned_scales
"""
from __future__ import annotations

import json
import os
import time

import numpy as np

from . import scales as S
from . import workloads as WL

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "data", "learned_scales.json")
SETTINGS = dict(k=3, steps=300, lr=0.02, seed=0, init="identity", noise="gaussian")


def model_layers(m):
    seen, out = set(), []
    for L in WL.LAYERS.values():
        if L.m != m:
            continue
        key = (L.cfg_id, L.layer_idx, L.G)
        if key in seen:  # the c4 standard / perturbed pair shares its weights
            continue
        seen.add(key)
        w = WL.make_w(L)
        cin = min(L.Cin, max(L.G, (256 // L.G) * L.G))
        cout = min(L.Cout, 32)
        out.append(dict(name=L.name, w=w[:cout, :cin], G=L.G, N=1, H=min(L.H, 14), W=min(L.W, 14)))
    return out


def main():
    rec = {"settings": dict(SETTINGS), "procedure": __doc__.split("\n\n")[1].replace("\n", " ")}
    for m in (4, 6):
        layers = model_layers(m)
        kk = min(SETTINGS["k"], len(layers))
        t0 = time.time()
        sb, sg, hist = S.learn_scales_model(m, layers, k=kk, steps=SETTINGS["steps"], lr=SETTINGS["lr"],
                                            seed=SETTINGS["seed"], init=SETTINGS["init"],
                                            noise=SETTINGS["noise"])
        rec[f"F({m},3)"] = {"s_B": sb, "s_G": sg, "layers": [L["name"] for L in layers], "k": kk,
                            "loss_first": round(hist[0], 3), "loss_last10": round(float(np.mean(hist[-10:])), 3)}
        print(f"F({m},3): {len(layers)} layers, k={kk}, {time.time() - t0:.1f} s, "
              f"-SQNR {hist[0]:.2f} -> {np.mean(hist[-10:]):.2f} dB", flush=True)
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
