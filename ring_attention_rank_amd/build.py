"""Build libra.so (HIP kernels + C-ABI host code) in-tree for gfx950.

Usage: python -m ring_attention_rank_amd.build   (or call build()).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libra.so")
SOURCES = [os.path.join(CSRC, "ra_kernels.hip"), os.path.join(CSRC, "ra_fast.hip"),
           os.path.join(CSRC, "ra_bwd.hip"),
           os.path.join(CSRC, "ra_host.cpp")]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out=LIB):
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the kernels never create NaN (empty rows are guarded), so max needs
        # no quieting; infinities stay honoured (masked scores are -inf)
        "-fno-honor-nans",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *SOURCES, "-o", out,
    ]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libra.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
