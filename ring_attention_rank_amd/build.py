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
SOURCES = [os.path.join(CSRC, n) for n in
           ("ra_kernels.hip", "ra_fast.hip", "ra_bwd_dq.hip", "ra_bwd_dkv.hip",
            "ra_bwd_generic.hip", "ra_noalloc.hip", "ra_calib.hip", "ra_host.cpp")]
# Per-source additions.  The backward dq kernel keeps its MFMA accumulators
# in VGPRs, where its VALU work reads them directly; the dk/dv kernel needs
# the AGPRs for its 256 accumulator values per lane and keeps the default.
EXTRA = {"ra_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the kernels never create NaN (empty rows are guarded), so max needs
        # no quieting; infinities stay honoured (masked scores are -inf)
        "-fno-honor-nans",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def compile_commands(objdir):
    """One hipcc -c command per source: (command, object path)."""
    out = []
    for src in SOURCES:
        name = os.path.basename(src)
        obj = os.path.join(objdir, name + ".o")
        out.append(([hipcc(), *flags(), *EXTRA.get(name, []), "-c", src, "-o", obj], obj))
    return out


def build(verbose=False):
    """Compile every source (in parallel) and link libra.so in place."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    with tempfile.TemporaryDirectory(prefix="ra_build_") as objdir:
        cmds = compile_commands(objdir)

        def run(c):
            if verbose:
                print(" ".join(c[0]), flush=True)
            return subprocess.run(c[0], capture_output=True, text=True)

        with ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(run, cmds))
        for (cmd, _), r in zip(cmds, results):
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed on {cmd[-3]}")
        tmp = LIB + ".tmp"
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
                *[o for _, o in cmds], "-o", tmp]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("linking libra.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
