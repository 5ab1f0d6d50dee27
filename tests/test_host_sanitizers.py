"""Host sanitizers over the C ABI (CPU only, no GPU needed).

The library is built with AddressSanitizer and UndefinedBehaviorSanitizer on its host
code (build.build_host_sanitized: the sanitizer flags go to the host compilation only),
and tests/test_abi.py runs against that build in a subprocess that preloads the
sanitizer runtime. Those tests drive every entry point's argument validation, workspace
sizing, plan query and error reporting, so an out-of-bounds host access, a use after
free, signed overflow or a misaligned access on those paths fails here.

The build takes about two minutes (the device code is compiled as usual); it is cached
in the temp directory under a hash of the sources and flags, so only the first run
after a source change pays for it.
"""

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from block_sparse_speculative_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _have_toolchain():
    try:
        B.hipcc()
        B.asan_runtime()
        return True
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not _have_toolchain(), reason="hipcc / ASan runtime not found")


def _sanitized_library():
    h = hashlib.sha256()
    for path in B.sources() + [os.path.join(B.INCLUDE, n) for n in sorted(os.listdir(B.INCLUDE))]:
        h.update(path.encode())
        h.update(open(path, "rb").read())
    for path in sorted(os.listdir(B.CSRC)):
        if path.endswith(".h"):
            h.update(open(os.path.join(B.CSRC, path), "rb").read())
    h.update(" ".join(B.HIPCC_FLAGS + B.SANITIZE_FLAGS).encode())
    d = os.path.join(tempfile.gettempdir(), f"sv_host_sanitized_{h.hexdigest()[:16]}")
    lib = os.path.join(d, "libsv.so")
    if not os.path.exists(lib):
        tmp = d + f".tmp{os.getpid()}"
        B.build_host_sanitized(os.path.join(tmp, "libsv.so"))
        try:
            os.replace(tmp, d)
        except OSError:            # another process finished the same build first
            shutil.rmtree(tmp, ignore_errors=True)
    return lib


def _env(lib):
    env = dict(os.environ)
    env.update(SV_LIBRARY=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_abi_tests_pass_under_address_and_undefined_behaviour_sanitizers():
    lib = _sanitized_library()
    env = _env(lib)
    # the subprocess loads the instrumented build, not the in-tree library
    probe = subprocess.run(
        [sys.executable, "-c",
         "import ctypes; from block_sparse_speculative_amd import _lib as L; L.lib(); "
         "print(L.LIB_PATH); ctypes.CDLL(None).__asan_init"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip().splitlines()[-1] == lib
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and " skipped" not in r.stdout.splitlines()[-1], r.stdout[-1000:]
