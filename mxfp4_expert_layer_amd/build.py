"""Build libft.so in-tree: HIP kernels for gfx950 with hipcc, host runtime with g++.

Usage: python -m mxfp4_expert_layer_amd.build   (or call build()).  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libft.so")
BUILD = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["ft_decode.hip", "ft_prefill.hip", "ft_debug.hip", "ft_scratch.hip"]
CXX_SOURCES = ["ft_api.cpp", "ft_host.cpp", "ft_ftw.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
CXX_FLAGS = [
    "-O3", "-fPIC", "-std=c++17", "-march=x86-64-v3", "-pthread",
    "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-fvisibility=hidden", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        objs.append(o)
        jobs.append([f"{ROCM}/bin/hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        objs.append(o)
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=4) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([f"{ROCM}/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
          "-pthread", f"-L{ROCM}/lib", "-lamdhip64", "-Wl,--no-undefined"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
