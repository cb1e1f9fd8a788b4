"""Build libw4a4.so (gfx950 only) in-tree with hipcc.

    python -m w4a4_block_scaled_amd.build [--jobs N]

Every source is compiled on each call (no staleness checks), then linked into
w4a4_block_scaled_amd/libw4a4.so next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libw4a4.so")
SOURCES = ["quantize.hip", "pack.hip", "gemm.hip", "solver.hip", "int4g64.hip", "int8g128.hip", "probe.hip",
           "capi.cpp"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 VALU ops (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep fp32 subnormals: quantization decisions must be exact for them
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source code generation options: the INT8 G=128 kernels apply each
# integer MFMA result on the VALU, so they take the MFMA results in ordinary
# vector registers (no copy out of the accumulation registers per result).
SOURCE_FLAGS = {"int8g128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if "warning" in warn:
        sys.stderr.write(warn + "\n")


def build(jobs: int = 4, verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


ASAN_DIR = os.path.join(HERE, "_build_asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libw4a4.so")


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime (to preload into an
    uninstrumented host process such as python)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_asan(jobs: int = 4, verbose: bool = False) -> str:
    """A variant of the library whose host code (the C ABI layer and the
    launchers) is built with AddressSanitizer; the device code is unchanged.
    Written to _build_asan/libw4a4.so; used with the runtime preloaded and
    W4A4_LIBRARY pointing at it."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    host_flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = [os.path.join(ASAN_DIR, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]

    def comp(src, obj):
        cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *host_flags, "-x", "hip", "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")

    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(comp, SOURCES, objs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", *objs, "-o", ASAN_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--asan", action="store_true", help="also build the AddressSanitizer host variant")
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    if a.asan:
        build_asan(a.jobs, verbose=True)
