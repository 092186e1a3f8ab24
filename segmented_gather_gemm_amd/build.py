"""Build libsgmv.so in-tree with hipcc for gfx950 (MI355X).

The library holds the C entry points (csrc/sgmv_api.cpp) and the gfx950
kernels (csrc/sgmv_kernels.hip) with the code object embedded; nothing is
compiled at run time.  Packed-fp32 VALU instructions are disabled for every
HIP translation unit.
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libsgmv.so")
SOURCES = [os.path.join(CSRC, "sgmv_api.cpp"), os.path.join(CSRC, "sgmv_kernels.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile libsgmv.so next to this file (always rebuilds); return its path."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; keep
    # the rest of the diagnostics.
    noise = "is not a recognized feature for this target"
    diag = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{diag}")
    if diag.strip() and verbose:
        print(diag)
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY} in {time.time() - t0:.1f}s", flush=True)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
