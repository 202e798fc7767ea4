"""Build ``libtav.so`` (the HIP library) in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in parallel, then linked.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtav.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l
                    and l.strip() != "1 warning generated." and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out and verbose:
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


# The host side of every source built with AddressSanitizer and
# UndefinedBehaviorSanitizer (the device code as usual): the argument checks,
# plans and host arithmetic behind the C ABI, checked by running the host
# tests against this build (TAV_LIBRARY=<path>, the sanitizer runtime
# preloaded). Not for GPU runs.
SAN_DIR = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "libtav_san.so")
SAN_FLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime():
    """The compiler's shared AddressSanitizer runtime, or None."""
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                          "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    found += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[0] if found else None


def build_sanitized() -> str:
    os.makedirs(SAN_DIR, exist_ok=True)

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        res = subprocess.run([HIPCC, *SAN_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr[-4000:]}")
        return obj
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources()))) as ex:
        objs = list(ex.map(one, sources()))
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan",
                    "-o", SAN_LIB, *objs], check=True)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
