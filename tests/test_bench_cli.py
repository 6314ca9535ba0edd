"""bench.py's command line on the CPU: more than one GPU is refused with a
message, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU only" in (res.stdout + res.stderr)
    assert res.stdout.strip() == "" or not res.stdout.strip().startswith("{")
