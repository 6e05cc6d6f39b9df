"""Build libsrp.so (the HIP kernels and the C ABI) in-tree for gfx950.

Each source compiles to its own object in parallel; the objects link into
selective_recompute_prefill_amd/libsrp.so, which the ctypes binding loads."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libsrp.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["abi.cpp", "k_gemm.hip", "k_select.hip", "k_attn.hip", "k_misc.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions stay off (the target feature is device-only; the host
# pass warns that it does not know it).
FLAGS = ["-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{p.stderr}")
    noise = [l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int | None = None, out: str = OUT, defines=()) -> str:
    """Compile every source and link libsrp.so (or `out`, with extra -D
    `defines`); returns its path."""
    build_dir = BUILD_DIR if out == OUT else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    extra = tuple(f"-D{d}" for d in defines)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{p.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
