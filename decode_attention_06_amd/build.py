"""Builds the HIP shared library libfd.so for gfx950, in-tree.

    python -m decode_attention_06_amd.build [-v] [--sanitized]

hipcc cross-compiles the device code for gfx950, so this runs without a GPU.
--sanitized also builds lib/libfd_sanitized.so: the same sources with the
host code instrumented by AddressSanitizer and UndefinedBehaviorSanitizer
(device code unchanged), for running the CPU-side tests under the
sanitizers (load it with the ASan runtime preloaded; see SANITIZER_RUNTIME).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libfd.so")
SANITIZED_LIB_PATH = os.path.join(LIB_DIR, "libfd_sanitized.so")

SOURCES = ["fd_kernels.hip", "fd_mfma.hip", "fd_bifurcated.hip", "fd_prefill.hip", "fd_noalloc.hip",
           "fd_validate.hip", "fd_api.cpp"]

# Packed-FP32 instructions stay disabled: ordinary float code only.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Host-only sanitizers: each flag goes to the host compilation alone.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sanitizer_runtime():
    """Path of the AddressSanitizer runtime matching hipcc's clang (to preload)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       stderr=subprocess.DEVNULL, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _compile_and_link(out_path, extra, tag, verbose):
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(build_dir, f"{src}{tag}.o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([hipcc()] + HIP_FLAGS + extra + ["-I", INCLUDE, "-I", CSRC, "-c"] + lang +
             [os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out_path + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out_path)
    return out_path


def build(verbose=False, sanitized=False):
    """Compile every source and link libfd.so (and, with sanitized=True,
    libfd_sanitized.so); raises on any compiler error."""
    os.makedirs(LIB_DIR, exist_ok=True)
    _compile_and_link(LIB_PATH, [], "", verbose)
    if sanitized:
        _compile_and_link(SANITIZED_LIB_PATH, SANITIZE_FLAGS, ".san", verbose)
    return LIB_PATH


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitized="--sanitized" in sys.argv))
