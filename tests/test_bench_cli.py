"""bench.py's command line on the CPU: more than one GPU is refused with a message, and the
workload list and options parse (no GPU work is started)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_workloads_and_options():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("headline", "decode-35b-a3b", "decode-35b-a3b-nvfp4", "decode-284b", "miss-path-284b",
              "prefill-753b", "prefill-753b-mxfp4"):
        assert w in r.stdout
    for opt in ("--layers", "--prefetch", "--residual-scale", "--disk-dir", "--ram-slots",
                "--split", "--adaptive", "--zipf-c", "--tokens"):
        assert opt in r.stdout
