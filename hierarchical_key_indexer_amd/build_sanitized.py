"""Build the library with AddressSanitizer and UndefinedBehaviorSanitizer on
its host code only (argument validation, size and plan computations, the
workspace carving, the Jacobi eigensolver); the gfx950 device code is built
as usual.  For CPU runs only:

    python -m hierarchical_key_indexer_amd.build_sanitized
    LSA_LIBRARY=hierarchical_key_indexer_amd/liblsa_san.so \\
    LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
        python -m pytest tests/test_abi_cpu.py tests/test_pca_host.py

The Python interpreter itself is not instrumented, so the sanitizer runtime is
preloaded and leak checking (which would report the interpreter's own
allocations) is off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

from .build_lib import ARCH, CSRC, FLAGS, HERE, HIPCC, SOURCES

OUT = os.path.join(HERE, "liblsa_san.so")
# each sanitizer flag goes to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src: str, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".san.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [HIPCC, *flags, *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan", *objs, "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    print(f"built {OUT}", flush=True)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
