"""Build libattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m attention_online_softmax_amd.build   (or build() from Python)

Every .hip/.cpp file under csrc/ is compiled by hipcc to an object, in
parallel, then linked into attention_online_softmax_amd/libattn.so; the
benchmark's measured-ceiling kernels (ceilings/) become libceilings.so.
Packed fp32 VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def device_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-file extra flags.  The d = 64 and 128 backward kernels run about 2 %
# faster under LLVM's iterative ILP scheduling strategy; the forward and
# decode kernels are fastest with the default one, and the d = 256 backward
# (bwd256.hip) spills less with it.
FILE_FLAGS = {
    "bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = ([hipcc()] + device_flags() + FILE_FLAGS.get(os.path.basename(src), []) + lang +
           ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    write_build_info()
    build_ceilings(verbose)
    return LIB


BUILD_INFO = os.path.join(PKG, "libattn.buildinfo.json")


def write_build_info() -> None:
    """The toolchain and flags libattn.so was built with, next to it, so
    that a run can record them without starting the compiler (a child
    program started from a process that uses the GPU is not always
    allowed)."""
    import hashlib
    import json
    r = subprocess.run([hipcc(), "--version"], capture_output=True, text=True)
    h = hashlib.sha256()
    with open(LIB, "rb") as f:
        h.update(f.read())
    info = {"hipcc": [ln for ln in r.stdout.splitlines() if ln.strip()][:2],
            "build_flags": [f.replace(ROOT, "<repo>") for f in device_flags()],
            "per_file_flags": FILE_FLAGS, "libattn_sha256_16": h.hexdigest()[:16]}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)


CEIL_SRC = os.path.join(PKG, "ceilings", "ceilings.hip")
CEIL_LIB = os.path.join(PKG, "ceilings", "libceilings.so")


def build_ceilings(verbose: bool = False) -> str:
    """The benchmark's measured-ceiling kernels (streaming read, MFMA loop),
    a library of their own that the attention library does not link."""
    tmp = CEIL_LIB + ".tmp"
    cmd = [hipcc()] + device_flags() + ["-shared", CEIL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEIL_SRC}:\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, CEIL_LIB)
    return CEIL_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
