"""Build libsgmv.so in-tree with hipcc for gfx950 (MI355X).

The library holds the C entry points (csrc/sgmv_api.cpp,
csrc/sgmv_shrink_api.cpp, with shared helpers in csrc/sgmv_host.cpp) and the
gfx950
kernels (csrc/sgmv_fast_ks*.hip, csrc/sgmv_generic.hip, built from
csrc/sgmv_device.h; csrc/sgmv_shrink_*.hip, built from csrc/sgmv_shrink.h;
both on csrc/sgmv_common.h)
with the code object embedded; nothing is
compiled at run time.  Packed-fp32 VALU instructions are disabled for every
HIP translation unit.

It also builds libsgmv_stream.so (csrc/sgmv_stream.hip), the benchmark's
streaming-bandwidth probe, which is not part of the operation, and
examples/sgmv_c_client, a plain C-ABI client of libsgmv (HIP runtime and
include/sgmv.h only) that the GPU tests run.
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
SOURCES = [os.path.join(CSRC, f) for f in
           ("sgmv_api.cpp", "sgmv_host.cpp", "sgmv_shrink_api.cpp", "sgmv_generic.hip", "sgmv_fast_ks0.hip", "sgmv_fast_ks1.hip",
            "sgmv_fast_ks2.hip", "sgmv_fast_ks4.hip", "sgmv_fast_ks8.hip",
            "sgmv_shrink_generic.hip", "sgmv_shrink_k1.hip", "sgmv_shrink_k2.hip",
            "sgmv_shrink_k4.hip", "sgmv_shrink_k8.hip", "sgmv_shrink_k16.hip",
            "sgmv_fused_api.cpp", "sgmv_fused_k1.hip", "sgmv_fused_k2.hip", "sgmv_fused_k4.hip",
            "sgmv_fused_k8.hip", "sgmv_valu.hip")]

STREAM_SOURCE = os.path.join(CSRC, "sgmv_stream.hip")
STREAM_LIBRARY = os.path.join(HERE, "libsgmv_stream.so")
CLIENT_SOURCE = os.path.join(HERE, "examples", "sgmv_c_client.cpp")
CLIENT = os.path.join(HERE, "examples", "sgmv_c_client")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, obj: str, flags) -> subprocess.CompletedProcess:
    cmd = [HIPCC, *FLAGS, *flags, "-c", src, "-o", obj]
    return cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _diagnostics(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature and says so; keep
    # the rest of the diagnostics.
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in text.splitlines() if noise not in l)


def build(verbose: bool = False, extra_flags=(), output: str = LIBRARY) -> str:
    """Compile every translation unit in parallel and link libsgmv.so, and
    build the streaming probe library (always rebuilds); return libsgmv's
    path."""
    t0 = time.time()
    stream_tmp = STREAM_LIBRARY + ".tmp%d" % os.getpid()
    stream_cmd = [HIPCC, *FLAGS, "-shared", STREAM_SOURCE, "-o", stream_tmp]
    stream_proc = subprocess.Popen(stream_cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                   text=True)
    tmpdir = output + ".objs%d" % os.getpid()
    os.makedirs(tmpdir, exist_ok=True)
    try:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd, proc = _compile(src, obj, [f for f in extra_flags if f != "-shared"])
            jobs.append((src, obj, cmd, proc))
        for src, obj, cmd, proc in jobs:
            out, _ = proc.communicate()
            if verbose:
                print(" ".join(cmd), flush=True)
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src} ({proc.returncode}):\n{_diagnostics(out)}")
            diag = _diagnostics(out)
            if diag.strip() and verbose:
                print(diag)
        tmp = output + ".tmp%d" % os.getpid()
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _, _ in jobs],
                "-o", tmp]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{_diagnostics(res.stdout + res.stderr)}")
        os.replace(tmp, output)
        out, _ = stream_proc.communicate()
        if stream_proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {STREAM_SOURCE}:\n{_diagnostics(out)}")
        os.replace(stream_tmp, STREAM_LIBRARY)
        if output == LIBRARY:
            # the C client links the in-tree library (found next to it at run time)
            client_tmp = CLIENT + ".tmp%d" % os.getpid()
            cmd = [HIPCC, "-O2", "-std=c++17", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
                   CLIENT_SOURCE, "-o", client_tmp, f"-L{HERE}", "-lsgmv",
                   "-Wl,-rpath,$ORIGIN/.."]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {CLIENT_SOURCE}:\n"
                                   f"{_diagnostics(res.stdout + res.stderr)}")
            os.replace(client_tmp, CLIENT)
    finally:
        if stream_proc.poll() is None:
            stream_proc.wait()
        for f in os.listdir(tmpdir):
            os.remove(os.path.join(tmpdir, f))
        os.rmdir(tmpdir)
    if verbose:
        print(f"built {output} in {time.time() - t0:.1f}s", flush=True)
    return output


if __name__ == "__main__":
    build(verbose=True)
