"""Build the HIP library libwino_q8_conv.so in-tree for gfx950.

hipcc compiles the kernels, the host plan and the C ABI (one object per
source, in parallel) and links them into a shared library next to this file. Numerics flags: no fp contraction (every fma
is written out), IEEE fp32 division, fp32 denormals kept, no packed fp32
instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwino_q8_conv.so")
SOURCES = ["wq8_kernels.hip", "wq8_hgemm.hip", "wq8_direct.hip", "wq8_noalloc.hip", "wq8_plan.cpp", "wq8_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the group dequantization reads every
    # int32 product once, and copies out of AGPRs cost a VALU op each
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link the library."""
    import concurrent.futures as cf
    import tempfile

    noise = "'-packed-fp32-ops' is not a recognized feature"
    with tempfile.TemporaryDirectory(prefix="wq8_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), file=sys.stderr)
            r = subprocess.run(cmd, capture_output=True, text=True)
            msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
            return src, obj, r.returncode, msgs

        with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
            results = list(ex.map(compile_one, SOURCES))
        for src, _, rc, msgs in results:
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{msgs}")
            if verbose and msgs.strip():
                print(msgs, file=sys.stderr)
        cmd = [HIPCC, *[f for f in FLAGS if f != "-c"], *[o for _, o, _, _ in results], "-o", LIB + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{msgs}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
