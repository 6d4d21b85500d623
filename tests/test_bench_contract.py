"""CPU checks of bench.py's command-line contract (no GPU needed): more than one GPU is refused
with a message and a non-zero exit status, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_counter_gate_follows_code_not_comments(tmp_path):
    """bench.py reports the traffic counters only while the attention kernel's code is the one
    they were taken on: its hash ignores comments and whitespace, not code."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) { return x + 1; }  /* tail */\n")
    b = tmp_path / "b.hip"
    b.write_text("// another header\n\nint f(int x) {\n  return x + 1;  // same code\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.code_hash(str(a)) == bench.code_hash(str(b))
    assert bench.code_hash(str(a)) != bench.code_hash(str(c))
