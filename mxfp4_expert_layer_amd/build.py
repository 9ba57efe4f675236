"""Build libft.so in-tree: HIP kernels for gfx950 with hipcc, host runtime with g++.

Usage: python -m mxfp4_expert_layer_amd.build   (or call build()).  Always recompiles.
       python -m mxfp4_expert_layer_amd.build --sanitize address|thread   (host runtime under
       ASan + UBSan or TSan, for the CPU tests; see build_sanitized).
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


SANITIZERS = {
    # kind -> g++ flags of the host runtime (the HIP objects are the ordinary ones)
    "address": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
    "thread": ["-fsanitize=thread"],
}


def sanitizer_runtime(kind: str) -> str:
    """The shared sanitizer runtime a process must preload to load the sanitized library."""
    name = {"address": "libasan.so", "thread": "libtsan.so"}[kind]
    return subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()


def build_sanitized(kind: str) -> str:
    """libft_<kind>.so: the host runtime (thread pool, LRU, host FFN, FTW files, C ABI) built
    by g++ with AddressSanitizer + UndefinedBehaviorSanitizer ("address") or ThreadSanitizer
    ("thread"), linked with the ordinary gfx950 kernel objects (sanitizers apply to host code
    only).  Load it with FT_LIB and the runtime from sanitizer_runtime() preloaded."""
    if kind not in SANITIZERS:
        raise ValueError(f"unknown sanitizer {kind!r}")
    os.makedirs(BUILD, exist_ok=True)
    hip_objs = []
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        hip_objs.append(o)
        if not os.path.exists(o):
            jobs.append([f"{ROCM}/bin/hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    objs = []
    flags = [f for f in CXX_FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                    *SANITIZERS[kind]]
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, f"{s}.{kind}.o")
        objs.append(o)
        jobs.append(["g++", *flags, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, jobs))
    out = os.path.join(BUILD, f"libft_{kind}.so")
    _run(["g++", "-shared", "-o", out + ".tmp", *objs, *hip_objs, *SANITIZERS[kind], "-pthread",
          f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64"])
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(sys.argv[sys.argv.index("--sanitize") + 1]))
    else:
        print(build(verbose="-v" in sys.argv))
