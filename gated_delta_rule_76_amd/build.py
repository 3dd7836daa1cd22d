"""Build libkda.so (the HIP library behind include/kda.h) for gfx950.

Each .hip translation unit is compiled with hipcc in parallel, then linked
into gated_delta_rule_76_amd/libkda.so; the same units compiled with
-DKDA_CHECKED=1 (bounds checks in every kernel) are linked into
libkda_checked.so, a debugging build; tests/c_abi_example, a plain-C caller of
the ABI, is linked against libkda.so.  The benchmark's calibration kernels
(csrc/calibrate.hip) go into a separate libkda_calibrate.so, outside the KDA
C ABI.  Usage: python -m gated_delta_rule_76_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
CHECKED_LIB = os.path.join(PKG, "libkda_checked.so")
CALIB_LIB = os.path.join(PKG, "libkda_calibrate.so")
ARCH = "gfx950"

SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip", "attnres.hip"]
CALIB_SOURCES = ["calibrate.hip"]

# -packed-fp32-ops off: every fp32 op stays scalar VALU (no v_pk_*_f32).
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkda.so")


def _compile(job) -> str:
    src, checked = job
    sub = os.path.join(BUILD, "checked") if checked else BUILD
    obj = os.path.join(sub, os.path.splitext(src)[0] + ".o")
    extra = ["-DKDA_CHECKED=1"] if checked else []
    cmd = [hipcc()] + CFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass reports the device-only feature flag as unknown: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


C_EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi_example.c")
C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi_example")


def _c_example() -> None:
    """The plain-C caller of the ABI that the GPU tests run (gcc, C99, the HIP
    runtime's C API; libkda.so found through an rpath relative to the binary)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C ABI example")
    tmp = C_EXAMPLE + f".tmp{os.getpid()}"
    cmd = [cc, "-O2", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), C_EXAMPLE_SRC, "-o", tmp, "-L", PKG, "-lkda",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../gated_delta_rule_76_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C ABI example failed to build:\n{r.stderr}")
    os.replace(tmp, C_EXAMPLE)


def build(verbose: bool = True) -> str:
    """Build libkda.so, its bounds-checked twin libkda_checked.so (the same
    sources with -DKDA_CHECKED=1) and libkda_calibrate.so."""
    os.makedirs(os.path.join(BUILD, "checked"), exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in SOURCES] + \
           [(s, False) for s in CALIB_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:2 * n], CHECKED_LIB)
    _link(objs[2 * n:], CALIB_LIB)
    _c_example()
    if verbose:
        print(f"built {LIB}, {CHECKED_LIB}, {CALIB_LIB} and {C_EXAMPLE}")
    return LIB


if __name__ == "__main__":
    build()
