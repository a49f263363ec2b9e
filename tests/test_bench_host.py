"""Host-side checks of bench.py that need no GPU: the one-GPU refusal and the
kernel-source hash that keys the recorded HBM traffic."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_code_text_ignores_comments_and_blank_lines():
    a = "int x = 1;  // a note\n\n/* block\n comment */\nint y = 2;\n"
    b = "int x = 1;\n// another note\nint y = 2;   \n"
    assert bench.code_text(a) == bench.code_text(b) == "int x = 1;\nint y = 2;"
    assert bench.code_text("int x = 1;\n") != bench.code_text("int x = 2;\n")


def test_kernel_source_hash_follows_code_not_comments():
    files = {}
    for name in bench.KERNEL_SOURCES:
        path = os.path.join(ROOT, "tiled_online_softmax_05_amd", "csrc", name)
        with open(path) as f:
            files[path] = f.read()
    h0 = bench.kernel_source_hash(lambda p: files[p])
    assert h0 == bench.kernel_source_hash()
    first = next(iter(files))
    commented = dict(files)
    commented[first] = "// an added comment line\n" + files[first]
    assert bench.kernel_source_hash(lambda p: commented[p]) == h0
    changed = dict(files)
    changed[first] = files[first] + "\nstatic int added_symbol;\n"
    assert bench.kernel_source_hash(lambda p: changed[p]) != h0

