"""Writes tests/golden/equalized_scales.json using only oracle/.

Data-free "equalizing" scales, an input for the SQNR checks and the benchmark
report (not the pages' learned values, which they do not print): for
i.i.d. zero-mean inputs and weights the Winograd-domain output Y[i][j] has a
standard deviation proportional to e_i e_j with e_i = |row i of B^T| |row i
of G|. Choosing s_B[i] = 1 / |row i of V^-T| and s_G[i] = 1 / |row i of V_nx3|
makes every e_i equal, which removes the cross-shaped spread of Y that the
pages blame for the collapse of standard scales (core claim, Fig. 3).
"""
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import transforms as T  # noqa: E402


def equalized(m):
    n = m + 2
    pts = T.standard_points(m)
    vinv = T.inverse(T.vandermonde(pts, n))
    vr = T.vandermonde(pts, 3)
    nb = [math.sqrt(sum(float(vinv[k][i]) ** 2 for k in range(n))) for i in range(n)]
    ngm = [math.sqrt(sum(float(vr[i][k]) ** 2 for k in range(3))) for i in range(n)]
    sb = [float(np.float32(1.0 / v)) for v in nb]
    sg = [float(np.float32(1.0 / v)) for v in ngm]
    return {"points": [str(p) for p in pts], "s_B": sb, "s_G": sg}


if __name__ == "__main__":
    out = {f"F({m},3)": equalized(m) for m in (4, 6)}
    with open(os.path.join(HERE, "equalized_scales.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
