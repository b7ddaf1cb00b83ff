"""CPU checks of bench.py's contract pieces that need no GPU: more than one GPU is refused with
a message, and the counter lookups' code hash ignores comments and whitespace but not code."""
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
    assert not r.stdout.strip()


def test_code_hash_ignores_comments_not_code():
    a = b"int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = b"int f(int x) {   return x + 1; }\n// another comment\n"
    c = b"int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)

