"""The host runtime under sanitizers (CPU only): libft's thread pool, LRU tables, host expert
FFN (AVX-512 and scalar paths), FTW reader and C ABI are rebuilt by g++ with AddressSanitizer
+ UndefinedBehaviorSanitizer and, separately, with ThreadSanitizer, and tests/test_lib_cpu.py
runs against each build in a child process with the sanitizer runtime preloaded.  Any report
fails the run (UBSan does not recover, TSan halts on its first report, ASan always aborts).
The GPU kernels are not sanitized (the ordinary gfx950 objects are linked in)."""
import os
import subprocess
import sys

import pytest

from mxfp4_expert_layer_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OPTIONS = {
    "address": {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1"},
    "thread": {"TSAN_OPTIONS": "halt_on_error=1:report_signal_unsafe=0"},
}


@pytest.mark.parametrize("kind", ["address", "thread"])
def test_host_runtime_under_sanitizer(kind):
    lib = build.build_sanitized(kind)
    env = dict(os.environ)
    # libstdc++ is preloaded too: python does not link it, and the sanitizer's exception
    # interceptors must find it at start-up
    env["LD_PRELOAD"] = " ".join([build.sanitizer_runtime(kind),
                                  subprocess.run(["g++", "-print-file-name=libstdc++.so"],
                                                 stdout=subprocess.PIPE, text=True,
                                                 check=True).stdout.strip()])
    env["FT_LIB"] = lib
    env.update(OPTIONS[kind])
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_lib_cpu.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=900)
    tail = r.stdout[-4000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stdout and "runtime error" not in r.stdout, tail
    assert " passed" in r.stdout, tail
