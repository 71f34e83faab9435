"""Host-side checks of bench.py's contract (no GPU work): one GPU only, and
the rocprofv3 summaries it writes name the command that made them."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")


def test_profile_summaries_carry_their_command():
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.endswith(".txt")]
    assert names
    for f in names:
        head = open(os.path.join(prof, f)).read(2048)
        assert "rocprofv3" in head and "bench.py" in head, f
