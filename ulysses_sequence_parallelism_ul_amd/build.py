"""Build libul.so (HIP kernels + C ABI) for gfx950 in-tree.

    python -m ulysses_sequence_parallelism_ul_amd.build

Every translation unit under csrc/ is compiled with hipcc in parallel into
_build/ and linked into ulysses_sequence_parallelism_ul_amd/libul.so.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libul.so")
PROBE_SRC = os.path.join(HERE, "probe", "mfma_rate.hip")
PROBE_LIB = os.path.join(HERE, "libul_probe.so")  # calibration probe (bench.py --mfma-ceiling), not the ABI

ARCH = "gfx950"
# Packed fp32 instructions are disabled for every HIP translation unit.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libul)")


def _compile(src, obj, verbose):
    cmd = [_hipcc()] + HIPCC_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc()] + [f for f in HIPCC_FLAGS if not f.startswith("--offload-arch")] + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose=False, jobs=None):
    """Compile every csrc/*.hip and csrc/*.cpp and link libul.so.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(8, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda p: _compile(p[0], p[1], verbose), zip(srcs, objs)))
    tmp = LIB_PATH + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel whose host stub was not emitted) fails the build
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    build_probe(verbose)
    return LIB_PATH


def build_probe(verbose=False):
    """Compile the MFMA-rate calibration probe into its own library, PROBE_LIB."""
    obj = os.path.join(BUILD_DIR, "probe_mfma_rate.o")
    _compile(PROBE_SRC, obj, verbose)
    tmp = PROBE_LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


# Host-side AddressSanitizer for the C ABI layer (argument validation, error
# strings, workspace arithmetic): the .cpp sources are compiled again with ASan
# and linked with the already-built kernel objects into a separate library.
# Device code is not instrumented (GPU ASan is not used here).
ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libul_asan.so")
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of the ASan runtime that a process loading ASAN_LIB must preload, or None."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def build_host_asan(verbose=False):
    """Build ASAN_LIB from csrc/*.cpp (ASan) plus the kernel objects of the last build()."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    cpps = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))
    kern = sorted(os.path.join(BUILD_DIR, f) for f in os.listdir(BUILD_DIR) if f.endswith(".hip.o"))  # not the probe
    if not kern:
        raise RuntimeError("no kernel objects in _build/; run build() first")
    objs = []
    for src in cpps:
        obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
        flags = [f for f in HIPCC_FLAGS if not f.startswith("--offload-arch")]
        cmd = [_hipcc()] + flags + ASAN_HOST_FLAGS + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
        objs.append(obj)
    cmd = ([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
            "-shared-libsan", "-o", ASAN_LIB] + kern + objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
