"""Host-side logic of bench.py (no GPU): the guard for more than one GPU and
the source digest that keeps stored hardware-counter figures tied to the
sources they were measured on (the bench reports null for them otherwise)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_source_digest_ignores_comments_not_code(tmp_path):
    b = _bench()
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) {\n    return x + 1;   // one more\n}\n/* block */\n")
    d0 = b.source_digest([str(a)])
    a.write_text("// header\nint f(int x) {\n  return x + 1; /* changed comment */\n}\n")
    assert b.source_digest([str(a)]) == d0
    a.write_text("int f(int x) {\n    return x + 2;\n}\n")
    assert b.source_digest([str(a)]) != d0

