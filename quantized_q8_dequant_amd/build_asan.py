"""Build a copy of the library whose host code is checked by AddressSanitizer.

The C-ABI runtime (argument checks, the workspace plan, the repack and launch
bookkeeping) is host code; this build instruments that host code only (each
sanitizer flag is scoped to the host pass), links it with the device objects
of the normal build, and writes it outside the package.  Load it under the
clang ASan runtime (`asan_runtime()` as LD_PRELOAD): the CPU tests of the
C ABI run against it that way.  No GPU is needed and no GPU run uses it.
"""

from __future__ import annotations

import glob
import os
import subprocess

from . import build as b


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime shipped with ROCm's LLVM."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return hits[-1]


HOST_SOURCES = ("runtime.cpp", "noalloc.hip")  # the sources with host logic beyond launches


def build_asan(out_dir: str) -> str:
    """Compile the host-logic sources with host-side ASan, link them with the
    other objects of the normal build, and return the library's path."""
    if not all(os.path.exists(os.path.join(b.BUILD, os.path.basename(p) + ".o"))
               for p in glob.glob(os.path.join(b.CSRC, "*.hip"))):
        b.build()
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for name in HOST_SOURCES:
        obj = os.path.join(out_dir, name + ".asan.o")
        cmd = [b._hipcc(), *b.DEVICE_FLAGS, "-g", *san, "-c", os.path.join(b.CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}:\n{r.stderr}")
        objs.append(obj)
    rest = [o for o in glob.glob(os.path.join(b.BUILD, "*.o"))
            if os.path.basename(o)[: -len(".o")] not in HOST_SOURCES]
    out = os.path.join(out_dir, "libqwen3q8_asan.so")
    cmd = [b._hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-fsanitize=address", "-shared-libasan",
           "-o", out, *objs, *rest]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return out
