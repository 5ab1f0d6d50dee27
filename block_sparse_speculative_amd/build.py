"""Build libsv.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m block_sparse_speculative_amd.build

Compiles every translation unit under csrc/ with hipcc (in parallel) and links
them into block_sparse_speculative_amd/libsv.so. Always rebuilds.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsv.so)")


def sources():
    out = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".hip") or name.endswith(".cpp"):
            out.append(os.path.join(CSRC, name))
    return out


# Build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code, for
# checking the host side of the C ABI (argument validation, workspace layout, error
# paths) on a machine without a GPU. Every sanitizer flag is given to the host
# compilation only (-Xarch_host); device code is built as usual, at -O1. The library
# leaves the sanitizer runtime unresolved; a process that loads it preloads
# libclang_rt.asan (asan_runtime()).
SANITIZE_FLAGS = [
    "-O1",
    "-g",
    "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (for LD_PRELOAD)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found ({path!r})")
    return path


def _link(cc, objs, out, extra):
    out_tmp = out + ".tmp"
    cmd = [cc, *extra, "-shared", "-fPIC", *objs, "-o", out_tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out_tmp, out)


def _build(out: str, flags, link_flags, verbose: bool) -> str:
    cc = hipcc()
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    srcs = sources()
    tmp = tempfile.mkdtemp(prefix="sv_build_")
    try:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))

        def one(so):
            src, obj = so
            cmd = [cc, *flags, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            return r.stderr

        with cf.ThreadPoolExecutor(jobs) as ex:
            logs = list(ex.map(one, zip(srcs, objs)))
        if verbose:
            for s, log in zip(srcs, logs):
                if log.strip():
                    print(f"[{os.path.basename(s)}]\n{log}", file=sys.stderr)
        _link(cc, objs, out, link_flags)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


def build(verbose: bool = False) -> str:
    return _build(LIB, HIPCC_FLAGS, [f"--offload-arch={ARCH}"], verbose)


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """Build the host-only ASan/UBSan library at `out` (see SANITIZE_FLAGS)."""
    flags = [f for f in HIPCC_FLAGS if f != "-O3"]
    return _build(out, [*flags, *SANITIZE_FLAGS], [f"--offload-arch={ARCH}"], verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
