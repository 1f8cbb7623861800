"""bench.py's command-line contract on the host (no GPU): more than one GPU
is refused with a message, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_path_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for opt in ["--workload", "--expcast", "--mma", "--p-format", "--v-format", "--rope",
                "--qk-hadamard", "--reuse-perm", "--gather"]:
        assert opt in r.stdout, opt
