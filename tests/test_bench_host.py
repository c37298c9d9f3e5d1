"""Host-side checks of bench.py's bookkeeping: the recorded HBM counters are
tied to the kernel source's code, not to its comments or layout; kernel names
map to stages; a request for more than one GPU is refused."""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sha_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    old = bench.KERNEL_SRCS
    bench.KERNEL_SRCS = [str(p)]
    try:
        return bench.kernel_source_sha()
    finally:
        bench.KERNEL_SRCS = old


def test_source_hash_ignores_comments_and_layout(tmp_path):
    base = "int f(int a) {\n    return a + 1;  // one more\n}\n"
    same = "/* header */\nint f(int a)\n{\n  return a + 1;\n}\n// trailer\n"
    other = "int f(int a) {\n    return a + 2;  // one more\n}\n"
    assert _sha_of(tmp_path, base) == _sha_of(tmp_path, same)
    assert _sha_of(tmp_path, base) != _sha_of(tmp_path, other)


def test_recorded_traffic_follows_source_hash():
    # counters come back only while they were taken on the code as it stands
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    current = rec["kernel_source_sha"] == bench.kernel_source_sha()
    for layer in rec["layers"]:
        for kernel, v in rec["layers"][layer].items():
            got = bench.recorded_traffic(layer, kernel)
            assert got == (v["bytes_per_launch"] if current else None)
    assert bench.recorded_traffic("no_such_layer", "stage1") is None


def test_stage_of_reads_the_template_arguments():
    # k_stage1<M, G, TPB, BMASK, VEC, XT, IQ, RH>: IQ marks the integer input stage
    s1 = "void wq8::k_stage1<6, 64, 4, 12285395915266489941ul, true, float, {iq}, {rh}>(x)"
    assert bench.stage_of(s1.format(iq="false", rh="true")) == "stage1"
    assert bench.stage_of(s1.format(iq="false", rh="false")) == "stage1"
    assert bench.stage_of(s1.format(iq="true", rh="false")) == "stage1_int"
    assert bench.stage_of("void wq8::k_stage1<6, 64, 4, 1ul, false, unsigned short, true, false>(x)") == "stage1_int"
    assert bench.stage_of("void wq8::k_fused23<6, 64, 4, false, float>(a)") == "stage23"
    assert bench.stage_of("void wq8::k_fused23w<6, 64, false, float>(a)") == "stage23"
    assert bench.stage_of("void wq8::k_stage2<32, 64, false>(a)") == "stage2"
    assert bench.stage_of("void wq8::k_hgemm<32, 5, 1, 4, false>(a)") == "stage2"
    assert bench.stage_of("void wq8::k_stage3<6, false, float>(a)") == "stage3"
    assert bench.stage_of("void wq8::k_weights<6, 64>(a)") is None


def test_more_than_one_gpu_is_refused():
    # the measurement is one GPU's; asking for more exits before any GPU work
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
