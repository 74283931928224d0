"""Build libpagedkv.so in-tree with hipcc for gfx950.

Usage: python paged_kv_cache_104_amd/build_lib.py [--jobs N]
(run it as a script: importing the package would load the library being rebuilt)
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.environ.get("PKV_BUILD_DIR", os.path.join(ROOT, "_build"))
LIB = os.environ.get("PKV_LIB_OUT", os.path.join(HERE, "libpagedkv.so"))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["errors.cpp", "block_manager.cpp", "prefix_rows.cpp", "cache_ops.hip", "decode.hip",
           "quest.hip", "read_probe.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-result"]
# device code: never emit packed-fp32 instructions (v_pk_*_f32)
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc"]


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.splitext(src)[0] + ".o")


def compile_one(src: str) -> str:
    path = os.path.join(CSRC, src)
    out = _obj(src)
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += HIP_FLAGS + os.environ.get("PKV_EXTRA_HIPFLAGS", "").split() + ["-x", "hip"]
    else:
        cmd += ["-x", "c++"]
    cmd += ["-c", path, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if noise not in ln and ln.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return out


# Host-only sources (no device code): the block manager, the unit builder of the
# shared-prefix decode and the error helpers.  build_host_sanitized() compiles them with
# g++ under AddressSanitizer and UndefinedBehaviorSanitizer into a library of their own.
HOST_SOURCES = ["errors.cpp", "block_manager.cpp", "prefix_rows.cpp"]
SAN_LIB = os.path.join(BUILD, "san", "libpagedkv_host_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host_sanitized(verbose: bool = False) -> str:
    """libpagedkv_host_san.so: the host sources under ASan + UBSan (g++).  Load it in a
    process started with the ASan runtime preloaded (sanitizer_env()) and with
    PKV_HOST_LIB pointing at it: the binding then exposes the host calls only."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    cxx = os.environ.get("CXX_HOST", "g++")
    srcs = [os.path.join(CSRC, f) for f in HOST_SOURCES]
    tmp = SAN_LIB + ".tmp"
    cmd = [cxx, "-std=c++17", "-shared", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"] + \
        SAN_FLAGS + srcs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_env(base=None) -> dict:
    """Environment for a child process that loads the sanitized host library: the ASan
    runtime preloaded (an uninstrumented python must load it first), leak checks off (the
    interpreter's own allocations are not ours to judge), stop at the first report."""
    env = dict(os.environ if base is None else base)
    cxx = os.environ.get("CXX_HOST", "g++")
    asan = subprocess.run([cxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PKV_HOST_LIB"] = SAN_LIB
    return env


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--sanitize", action="store_true",
                    help="build the host-only ASan/UBSan library instead (also PKV_SANITIZE=1)")
    args = ap.parse_args()
    if args.sanitize or os.environ.get("PKV_SANITIZE") == "1":
        build_host_sanitized(verbose=True)
    else:
        build(args.jobs, verbose=True)
