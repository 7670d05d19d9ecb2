"""Host-side rules of bench.py, on the CPU.

* main_kernel_name restates the library's decode dispatch (the kernel whose launches the
  roofline times): the split kernel for bf16/fp16 with head_dim 64/128 on blocks of 16 << j
  tokens and head_dim 256 on 16-token blocks (at most 2048 sequences), the per-partition MFMA
  kernel beyond 2048 sequences on 16-token blocks, the VALU kernel for everything else.
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


@pytest.mark.parametrize("args,kernel", [
    (("bf16", 128, 1, 64, 16), "decode_split_kernel"),
    (("f16", 64, 16, 2048, 16), "decode_split_kernel"),
    (("bf16", 128, 4, 2049, 16), "decode_mfma_kernel"),
    (("bf16", 128, 4, 64, 32), "decode_split_kernel"),
    (("bf16", 64, 8, 64, 1024), "decode_split_kernel"),
    (("bf16", 128, 4, 4096, 32), "decode_generic_kernel"),
    (("bf16", 128, 4, 64, 48), "decode_generic_kernel"),
    (("bf16", 128, 4, 64, 8), "decode_generic_kernel"),
    (("bf16", 256, 4, 64, 16), "decode_split_kernel"),
    (("bf16", 256, 4, 64, 32), "decode_generic_kernel"),
    (("bf16", 256, 4, 4096, 16), "decode_generic_kernel"),
    (("bf16", 128, 32, 64, 16), "decode_generic_kernel"),
    (("bf16", 96, 4, 64, 16), "decode_generic_kernel"),
    (("f32", 128, 1, 64, 16), "decode_generic_kernel"),
])
def test_main_kernel_name(args, kernel):
    assert bench.main_kernel_name(*args) == kernel


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
