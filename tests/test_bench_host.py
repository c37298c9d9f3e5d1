"""Host-side checks of bench.py's bookkeeping: the recorded HBM counters are
tied to the kernel source's code, not to its comments or layout."""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sha_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    old = bench.KERNEL_SRC
    bench.KERNEL_SRC = str(p)
    try:
        return bench.kernel_source_sha()
    finally:
        bench.KERNEL_SRC = old


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
    layer = "c2_f6_n32_c64_56x56_g64"
    for kernel, v in rec["layers"][layer].items():
        got = bench.recorded_traffic(layer, kernel)
        assert got == (v["bytes_per_launch"] if current else None)
    assert bench.recorded_traffic("no_such_layer", "stage1") is None
