"""Build libmscan.so (HIP, gfx950) in-tree with hipcc.

Usage: python associative_scan_amd/build.py   (or call build()); run as a
script, since importing the package needs the library this builds.
Each source compiles to an object under associative_scan_amd/_build/, in
parallel, then links into associative_scan_amd/libmscan.so. A second library,
libmscan_stress.so, is the same code with MSCAN_RACE_STRESS defined (a
pseudo-random pause before every look-back publish); only the race-stress
tests load it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmscan.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("MSCAN_ARCH", "gfx950")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

# Packed fp32 VALU ops are disabled: the kernels get no v_pk_{add,mul,fma}_f32.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]


# Every source compiles in well under a minute; a compile that runs past this
# is a compiler problem and fails the build instead of stalling it.
COMPILE_TIMEOUT_S = 900


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; libmscan needs ROCm's hipcc to build")
    return h


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


STRESS_OUT = os.path.join(HERE, "libmscan_stress.so")
STRESS_FLAGS = ["-DMSCAN_RACE_STRESS"]


def _compile(job) -> str:
    src, variant = job
    d = os.path.join(BUILD, variant) if variant else BUILD
    obj = os.path.join(d, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *(STRESS_FLAGS if variant == "stress" else []), "-c", src, "-o", obj]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=COMPILE_TIMEOUT_S)
    except subprocess.TimeoutExpired as e:
        raise RuntimeError(f"hipcc did not finish {src} within {COMPILE_TIMEOUT_S} s") from e
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln and "(ignoring feature)" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, stress: bool = True) -> str:
    """Compile every source under csrc/ and link libmscan.so (and the race-stress
    build libmscan_stress.so); returns the path of libmscan.so."""
    variants = ["", "stress"] if stress else [""]
    for v in variants:
        os.makedirs(os.path.join(BUILD, v) if v else BUILD, exist_ok=True)
    srcs = sources()
    jobs = [(src, v) for v in variants for src in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(srcs)], OUT)
    if stress:
        _link(objs[len(srcs):], STRESS_OUT)
    if verbose:
        print(f"built {OUT}" + (f" and {STRESS_OUT}" if stress else ""))
    return OUT


if __name__ == "__main__":
    build(verbose=True)
