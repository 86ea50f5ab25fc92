"""Build libw4_hostsan.so: the library with its host code under AddressSanitizer
and UndefinedBehaviorSanitizer (the argument checks, the dispatch, the
launch wrappers).  The gfx950 device code is built exactly as by build.py.

For CPU-only checks of the host side (the GPU code is not instrumented, and
GPU sanitizers are not used).  Run the host tests against it with the clang
ASan runtime preloaded:

    python int4_weight_quantized_amd/build_hostsan.py
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \\
    ASAN_OPTIONS=detect_leaks=0 W4_LIB=$PWD/int4_weight_quantized_amd/libw4_hostsan.so \\
    python -m pytest tests/test_abi_host.py -q
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
from int4_weight_quantized_amd import build as B  # noqa: E402

OUT = os.path.join(HERE, "libw4_hostsan.so")
OBJ = os.path.join(HERE, "_build", "hostsan")
# host-side only: each sanitizer flag is preceded by -Xarch_host
HOST_SAN = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"):
    HOST_SAN += ["-Xarch_host", flag]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [B._hipcc()] + B.CFLAGS + HOST_SAN + lang + ["-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    cmd = [B._hipcc(), "-shared", f"--offload-arch={B.ARCH}", "-o", OUT] + objs
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    print(build())
