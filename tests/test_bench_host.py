"""bench.py's host-side bookkeeping (no GPU): the measured-traffic table is
tied to the code of the kernels it was measured on."""

import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))

import bench  # noqa: E402


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {  // the step\n    return x + 1; /* one */\n}\n"
    b = "/* header */\nint f(int x) {\n  return x + 1;\n}  // trailing\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("x + 1", "x + 2"))


def test_every_traffic_entry_names_a_kernel_and_summary():
    root = os.path.dirname(os.path.abspath(bench.__file__))
    for key, entry in bench.MEASURED_TRAFFIC.items():
        assert entry["kernel"] in bench.KERNEL_SOURCES, key
        assert entry["bytes"] > 0, key
        assert os.path.exists(os.path.join(root, entry["summary"])), key
        assert len(entry["sources_sha256"]) == 64, key
