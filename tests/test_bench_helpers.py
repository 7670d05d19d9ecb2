"""Host-side rules of bench.py, on the CPU.

* the kernel the roofline times is named by the library itself (paged_attention_decode_kernel,
  tested in test_abi.py), not restated here.
* kernel_code_hash ignores comments and blank lines, and nothing else.
* bench.py measures one GPU: asking for more exits with status 2 before touching a device.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_kernel_code_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;\n}\n")
    b.write_text("// header\n/* block\n comment */\nint f(int x) {  // inline\n\n  return x + 1;\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_code_hash(a) == bench.kernel_code_hash(b)
    assert bench.kernel_code_hash(a) != bench.kernel_code_hash(c)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
