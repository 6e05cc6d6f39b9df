"""Debug build of libsrp with AddressSanitizer on its host code.

The C ABI's host code (argument checks, workspace arithmetic, rotary tables, the
stack executor) is compiled with the sanitizer; the GPU kernels are compiled as in
the regular build (the sanitizer applies to host code only). The result,
libsrp_asan.so next to libsrp.so, is for host-side checks on the CPU: load it
through the binding (SRP_LIB) in a process that preloads the clang ASan runtime
(asan_runtime()). It is not used by any GPU run."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from . import build as B

OUT = os.path.join(B.PKG, "libsrp_asan.so")
BUILD_DIR = os.path.join(B.PKG, "_build_asan")
# host-side instrumentation only: every sanitizer flag is scoped to the host pass
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc's compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def build_asan(out: str = OUT) -> str:
    """Compile every source (abi.cpp with host ASan) and link `out`; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)

    def one(src):
        return B._compile(src, BUILD_DIR, tuple(HOST_ASAN) if src.endswith(".cpp") else ())

    with ThreadPoolExecutor(len(B.SOURCES)) as ex:
        objs = list(ex.map(one, B.SOURCES))
    tmp = out + ".tmp"
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{p.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_asan())
