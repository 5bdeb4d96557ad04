"""Build the host-sanitized library and the C-ABI checker of tests/abi_sanitize.

Every source of the library is compiled again with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code only (each -fsanitize= behind
-Xarch_host; the gfx950 device code is built as usual) into
eagle_draft_head_amd/_asan/libeagle3_asan.so, and abi_check.cpp is linked against
it into eagle_draft_head_amd/_asan/abi_check.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
from eagle_draft_head_amd import build as B  # noqa: E402

OUT = os.path.join(ROOT, "eagle_draft_head_amd", "_asan")
LIB = os.path.join(OUT, "libeagle3_asan.so")
EXE = os.path.join(OUT, "abi_check")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}", "-Wall", "-Wno-unused-function",
         "-Wno-unused-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(" ".join(cmd) + "\n" + msgs)


def build() -> str:
    os.makedirs(OUT, exist_ok=True)

    def obj(src):
        o = os.path.join(OUT, os.path.basename(src) + ".o")
        _run([B.HIPCC] + FLAGS + SAN + ["-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", o])
        return o

    with ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(obj, B.SOURCES))
    _run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC"] + SAN + ["-o", LIB] + objs)
    _run([B.HIPCC] + FLAGS + SAN + ["-x", "hip", os.path.join(HERE, "abi_check.cpp"), "-x", "none", LIB,
                                     "-o", EXE, f"-Wl,-rpath,{OUT}"])
    return EXE


if __name__ == "__main__":
    print(build())
