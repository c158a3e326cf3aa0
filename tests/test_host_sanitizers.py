"""The host half of the C ABI (validation, planners, marshalling, error paths)
under AddressSanitizer and UndefinedBehaviorSanitizer.

The two host sources are compiled with g++ and the sanitizers into a
host-only library (the device launchers replaced by stubs that return an
error, tests/sanitize/launch_stubs.cpp), and the host ABI tests run against
it in a child process with the ASan runtime preloaded.  Any sanitizer report
fails the run.  No GPU is involved."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_compressed_mla_amd", "csrc")


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("g++") is None or _runtime("libasan.so") is None,
                    reason="g++ with the ASan runtime is not available")
def test_host_abi_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "libcsmla_host_asan.so")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               os.path.join(CSRC, "csmla_host.cpp"), os.path.join(CSRC, "csmla_indexer_host.cpp"),
               os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ)
        env.update(CSMLA_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            "tests/test_abi_host.py", "tests/test_abi_indexer_host.py"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert " passed" in out
