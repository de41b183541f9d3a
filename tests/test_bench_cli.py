"""bench.py's command line on a host without a GPU (CPU only): more than one
GPU is refused with a message, and the source hashes that tie recorded
counter data to a build cover every kernel family bench.py reports."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_kernel_source_hashes():
    for prefix in ("decode_", "prefill_", "copy_"):
        h = bench.kernel_source_hash(prefix)
        assert len(h) == 64 and h == bench.kernel_source_hash(prefix)
    assert bench.kernel_source_hash("decode_") != bench.kernel_source_hash("prefill_")


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {  // one\n  return x + 1; /* two\n three */\n}\n"
    b = "// header\nint f(int x) {\n\n  return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
