"""Build the KDA HIP library for gfx950 in-tree: chunkwise_kimi_delta_amd/libkda_mi355x.so.

Usage: python -m chunkwise_kimi_delta_amd.build   (or call build()).
Every call recompiles.  Needs hipcc (cross-compiles without a GPU).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libkda_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["kda_api.cpp", "kda_intra.hip", "kda_scan.hip", "kda_merge.hip", "kda_recurrent.hip",
           "kda_noalloc.hip", "kda_bwd.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the KDA library needs ROCm's hipcc to build")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            # keep packed fp32 instructions out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc] + _flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{msg}")
        if verbose and msg.strip():
            print(msg)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-only sanitizer build of the C ABI (kda_api.cpp with stand-in launchers):
# the validation, planning and error paths under AddressSanitizer and
# UndefinedBehaviorSanitizer, for CPU tests on a machine without a GPU.  Each
# -fsanitize applies to the host pass only; no device code is built.
SAN_LIB_PATH = os.path.join(HERE, "_build", "libkda_host_asan.so")
_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized() -> str:
    hipcc = _hipcc()
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in ("kda_api.cpp", "kda_host_stubs.cpp"):
        obj = os.path.join(out_dir, src + ".san.o")
        cmd = [hipcc, "--cuda-host-only", "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE,
               "-I", CSRC] + _SAN + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build of {src} failed:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    r = subprocess.run([hipcc, "-shared", "-fPIC"] + _SAN + objs + ["-o", SAN_LIB_PATH],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the sanitizer build failed:\n{r.stdout}{r.stderr}")
    return SAN_LIB_PATH


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that the sanitizer build links against."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the clang AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
