"""Host-side pieces of the benchmark: the kernel-source hash that ties the
stored rocprofv3 traffic figures to the kernels they were measured on."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_tokens_ignore_comments_and_layout():
    a = "int f(int x) {  // add one\n  return x + 1; /* fast\n path */ }\n"
    b = "int f(int x)\n{\n  return x + 1;\n}\n// trailing note\n"
    assert bench.code_tokens(a) == bench.code_tokens(b) == "int f(int x) { return x + 1; }"


def test_code_tokens_see_code_changes():
    assert bench.code_tokens("a = b + c; // x") != bench.code_tokens("a = b - c; // x")
    assert bench.code_tokens("s = 1 /* one */;") != bench.code_tokens("s = 2 /* one */;")


def test_stored_traffic_files_name_a_source_hash():
    for name in sorted(f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("traffic_")):
        d = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert len(d["kernel_source_sha"]) == 16
        assert d["fetch_size_kib_per_dispatch"] > 0 and d["write_size_kib_per_dispatch"] > 0
    for e in bench.ENGINE_SOURCES:
        assert len(bench.kernel_source_hash(e)) == 16
