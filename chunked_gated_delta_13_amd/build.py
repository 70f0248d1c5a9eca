"""Build libkda.so (HIP, gfx950) in-tree.

Every .hip translation unit is compiled in parallel with hipcc for gfx950, then
linked with the host API into ``libkda.so`` next to this file.  Packed fp32
arithmetic is disabled for all device code (``-packed-fp32-ops`` off).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
PEAKS_LIB = os.path.join(HERE, "libkda_peaks.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """libkda.so from csrc/*.hip and csrc/*.cpp, and the benchmark's bandwidth probes
    (libkda_peaks.so, from csrc/bench/) beside it."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))
    probe_srcs = sorted(os.path.join(CSRC, "bench", f) for f in os.listdir(os.path.join(CSRC, "bench"))
                        if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
        probe_objs = list(ex.map(_compile, probe_srcs))
    _link(objs, LIB)
    _link(probe_objs, PEAKS_LIB)
    if verbose:
        print(f"built {LIB} and {PEAKS_LIB}")
    return LIB


def build_sanitized(out_dir: str | None = None) -> str:
    """libkda.so with its host code (argument validation, planning, launch set-up in
    kda_api.cpp) built by g++ under AddressSanitizer and UndefinedBehaviorSanitizer, linked with
    the device objects of the regular build (run build() first).  Load it with gcc's libasan and
    libubsan preloaded; the device code is unchanged."""
    out_dir = out_dir or os.path.join(BUILD_DIR, "asan")
    os.makedirs(out_dir, exist_ok=True)
    probes = {os.path.basename(f) + ".o" for f in os.listdir(os.path.join(CSRC, "bench"))}
    objs = sorted(os.path.join(BUILD_DIR, f) for f in os.listdir(BUILD_DIR)
                  if f.endswith(".hip.o") and f not in probes)
    if not objs:
        raise RuntimeError("no device objects in _build: run build() first")
    api_obj = os.path.join(out_dir, "kda_api.o")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{INCLUDE}", f"-I{CSRC}", "-c",
           os.path.join(CSRC, "kda_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(out_dir, "libkda.so")
    cmd = ["g++", "-shared", *san, "-o", lib, api_obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    if sys.argv[1:] == ["sanitized"]:
        print(build_sanitized())
    else:
        build(verbose=True)
    sys.exit(0)
