"""Host-sanitized build of libloki.so for CPU-side checks of the C ABI.

The host code of the C ABI (argument validation, workspace planning, the
launch sequence) is rebuilt with AddressSanitizer and UndefinedBehavior-
Sanitizer; device code is unchanged (the sanitizer flags apply to the host
compilation only).  The kernel translation units are linked from the normal
build's objects (``_build/*.o``, made by ``build.build()``).  The result is
``_build/libloki_hostsan.so``; load it with the ASan runtime preloaded
(``asan_runtime()``) and ``LOKI_LIBRARY`` pointing at it.
"""

from __future__ import annotations

import glob
import os
import subprocess

from . import build as b

OUT = os.path.join(b.BUILD, "libloki_hostsan.so")
# each host-only sanitizer flag directly after -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return cands[-1]


def build_sanitized() -> str:
    os.makedirs(b.BUILD, exist_ok=True)
    others = [os.path.join(b.BUILD, s + ".o") for s in b.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        b.build(verbose=False)
    obj = os.path.join(b.BUILD, "api.hip.hostsan.o")
    cmd = [b.hipcc(), *b.COMMON_FLAGS, "-g", *SAN, "-c", os.path.join(b.SRC, "api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for api.hip (sanitized):\n{r.stdout}\n{r.stderr}")
    # the sanitizer symbols stay undefined in the library: the preloaded runtime provides them
    cmd = [b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", OUT, obj, *others]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (sanitized):\n{r.stdout}\n{r.stderr}")
    return OUT


if __name__ == "__main__":
    print(build_sanitized())
