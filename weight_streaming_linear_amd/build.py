"""Build libwsl.so (the gfx950 HIP library) in-tree with hipcc.

Run as ``python -m weight_streaming_linear_amd.build`` or call ``build()``.
Every call compiles from source; nothing is cached between calls.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libwsl.so")

HIP_SOURCES = ["api.hip", "pack.hip", "gemv.hip", "gemm.hip", "embed.hip", "ring.hip", "probe.hip"]
CXX_SOURCES = ["validate.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # keep packed-fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def build(verbose=False):
    """Compile every source and link libwsl.so next to this file; returns its path."""
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(out_dir, src.replace(".cpp", ".host.o"))
        cmd = [hipcc, "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    # an unresolved symbol (e.g. a kernel's host launch stub that was not emitted) only
    # shows when the library is loaded: load it here, in a child process, before installing
    r = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1])", tmp],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("built library does not load: " + r.stdout.strip()[-2000:])
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError("build failed: " + " ".join(cmd))
    if verbose and r.stdout.strip():
        # the host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
