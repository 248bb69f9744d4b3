"""Host-side sanitizer build of the library, for CPU checks of the host code.

Every source is compiled as in build.py, but the host half of each
compilation is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(the flags go to the host compiler only; device code is built exactly as in
the product library). The result, _build/asan/libnanochat_asan.so, is loaded
by a Python process started with the sanitizer runtime preloaded, which runs
the host-only ABI tests against it: config validation, layout and workspace
planning, argument checks before any launch. No GPU is needed or used.

    python -m dense_gpt_pretraining_nanochat_amd.sanitize   # build + print the runtime path
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from . import build as b

ASAN_DIR = os.path.join(b.BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libnanochat_asan.so")
# host-only instrumentation: each sanitizer flag directly after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def _compile(src):
    obj = os.path.join(ASAN_DIR, src + ".o")
    cmd = [b._hipcc(), *b.COMMON, *b.DEVICE_FLAGS, *HOST_SAN, "-c", os.path.join(b.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed on {src}:\n{r.stderr}")
    return obj


def runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(b._hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_asan() -> str:
    os.makedirs(ASAN_DIR, exist_ok=True)
    srcs = b.sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = ASAN_LIB + ".tmp"
    cmd = [b._hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fno-gpu-sanitize",
           "-fsanitize=address,undefined", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer link failed:\n" + r.stderr)
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build_asan())
    print(runtime())
    sys.exit(0)
