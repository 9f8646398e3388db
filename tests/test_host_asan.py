"""The C-ABI tests again, against a build whose host-side ABI layer (argument
checks, overlap tests, error strings, workspace arithmetic) is compiled with
AddressSanitizer, in a child process with the ASan runtime preloaded.  CPU
only: every call fails a check before anything touches a GPU."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_asan():
    from ulysses_sequence_parallelism_ul_amd import build as B

    if shutil.which(B._hipcc()) is None and not os.path.exists(B._hipcc()):
        pytest.skip("hipcc not available")
    if not os.path.isdir(B.BUILD_DIR) or not any(f.endswith(".hip.o") for f in os.listdir(B.BUILD_DIR)):
        pytest.skip("kernel objects not built (run build() first)")
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("ASan runtime not found")
    lib = B.build_host_asan()
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UL_LIBRARY_PATH=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
