"""Build libmk.so (the persistent decode megakernel and its C ABI) for gfx950 with hipcc.

Run ``python -m decode_megakernel_03_amd.build``; the library lands next to this file. Every HIP
translation unit is compiled with packed-FP32 instructions disabled and without implicit FMA
contraction (the kernels fuse multiply-adds explicitly where the method allows it).
"""

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = ["mk_kernel.hip", "mk_host.cpp", "mk_server.cpp"]


def build(verbose=True, csrc=CSRC, out=LIB):
    """Compile the sources in `csrc` (default: this package's csrc/) into the shared library `out`."""
    common = [c if c != CSRC else csrc for c in COMMON]
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = [] if src.endswith(".hip") else ["-x", "hip"]
            cmd = [HIPCC] + common + lang + ["-c", os.path.join(csrc, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((subprocess.Popen(cmd), cmd))
            objs.append(obj)
        for pr, cmd in procs:
            if pr.wait() != 0:
                raise RuntimeError("compile failed: " + " ".join(cmd))
        tmp_lib = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
