"""Build libddt with AddressSanitizer and UndefinedBehaviorSanitizer on its
host code (argument validation, planning, launch set-up) into
_build/sanitize/libddt_sanitize.so.  The device code is compiled exactly as
in the regular build; only the host side carries the sanitizers (each
-fsanitize= flag is scoped to the host pass with -Xarch_host).

    python tests/sanitize/build_sanitized.py      # prints the library path
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from block_diffusion_draft_vocab_amd import build as B  # noqa: E402

OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "libddt_sanitize.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def runtime() -> str:
    """Path of the ASan runtime to preload into an uninstrumented Python."""
    clang = os.path.join(os.path.dirname(B._hipcc()), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True, check=True).stdout.strip()


def build() -> str:
    hipcc = B._hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)

    def one(src):
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *B.FLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(B.SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, B.SOURCES))
    cmd = [hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan",
           *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
