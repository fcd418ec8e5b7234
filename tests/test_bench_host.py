"""Host-side pieces of bench.py (CPU only): the stage-1 source hash that
decides whether the committed HBM counter summary still applies (bench.py
reports the traffic as null when it does not)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_sha_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // add one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    base = bench.kernel_sha()
    src.write_text("// a new header comment\nint f(int x) {\n\n  return x + 1;  // add one, reworded\n}\n")
    assert bench.kernel_sha() == base
    src.write_text("int f(int x) {\n  return x + 2;  // add one\n}\n")
    assert bench.kernel_sha() != base

