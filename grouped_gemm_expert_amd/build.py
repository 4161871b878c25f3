"""Build libmoe.so (the HIP library behind include/moe.h) in-tree for gfx950.

Usage:  python -m grouped_gemm_expert_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmoe.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["api.cpp", "router.hip", "permute.hip", "gemm.hip", "dense.hip", "elementwise.hip",
           "mx.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# No packed fp32 instructions: keep every fp32 op scalar on this target.
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


# Host-code sanitizers (a CPU test build of the host layer; device code is
# built as always): every -fsanitize= goes to the host pass only.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str, verbose: bool, build_dir: str, defines, extra=()) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = ([HIPCC] + COMMON + list(extra) + [f"-D{d}" for d in defines]
           + ["-c", os.path.join(CSRC, src), "-o", obj])
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 7, out: str = OUT, defines=(),
          sanitize_host: bool = False) -> str:
    """Compile every source and link `out`.  `defines` (NAME=VALUE strings) and
    `out` exist for building variants outside the package; sanitize_host
    builds the host code with AddressSanitizer and UndefinedBehaviorSanitizer
    (for CPU tests of the host layer; the process must preload clang's ASan
    runtime)."""
    if sanitize_host and out == OUT:
        raise ValueError("the sanitizer build goes to its own path")
    build_dir = BUILD_DIR if out == OUT else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    extra = HOST_SANITIZE if sanitize_host else ()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines, extra), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if sanitize_host:
        cmd += ["-shared-libsan"] + HOST_SANITIZE
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
