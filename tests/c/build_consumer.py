"""Build the C99 consumer of libsv.so (tests/c/sv_consumer.c) with gcc.

The program and this header-only build are test infrastructure: the consumer links the
in-tree libsv.so (found through an $ORIGIN-relative run path, so the tree can move) and
the HIP runtime, and compiles with -std=c99 -pedantic -Werror so that include/sv.h is
checked as C.
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "block_sparse_speculative_amd")
SRC = os.path.join(HERE, "sv_consumer.c")
OUT = os.path.join(HERE, "sv_consumer")


def rocm() -> str:
    for cand in (os.environ.get("ROCM_PATH"), "/opt/rocm"):
        if cand and os.path.exists(os.path.join(cand, "include", "hip", "hip_runtime_api.h")):
            return cand
    raise RuntimeError("ROCm headers not found")


def build(out: str = OUT) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no C compiler")
    r = rocm()
    rel = os.path.relpath(PKG, os.path.dirname(os.path.abspath(out)))
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(r, "include"),
           "-I", os.path.join(ROOT, "include"), SRC, "-o", out,
           "-L", os.path.join(r, "lib"), "-lamdhip64", "-L", PKG, "-l:libsv.so", "-lm",
           f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{os.path.join(r, 'lib')}"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"consumer build failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return out


if __name__ == "__main__":
    print(build())
