"""Host-side checks of bench.py (no GPU): the one-GPU contract and the kernel hash that
decides whether a stored HBM-traffic measurement still describes the decode kernel."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert '"metric"' not in r.stdout


def test_kernel_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// header\nint f(int x) {\n  return x + 1;  // add one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h0 = bench.kernel_hash()
    src.write_text("// another header\n\nint f(int x) {\n  // a new note\n  return x + 1;\n}\n")
    assert bench.kernel_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_hash() != h0
