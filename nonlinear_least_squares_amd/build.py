"""Builds the gfx950 shared libraries in-tree with hipcc.

``python -m nonlinear_least_squares_amd.build`` compiles ``libba.so`` (the
fp64 bundle-adjustment LM iteration), ``libdba.so`` (the fp32 dense
frame-graph variant) and ``libpgo.so`` (fp64 pose-graph optimisation) next
to this file.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ARCH = os.environ.get("BA_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # Contract only within one source expression, so the same expression
    # rounds the same way in every kernel that inlines it.
    "-ffp-contract=on",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

LIBS = {
    "libba.so": ["ba_kernels.hip", "ba_dense.hip", "ba_backward.hip", "ba_dogleg.hip", "ba_noalloc.hip",
                 "ba_capi.hip"],
    "libdba.so": ["dba_kernels.hip"],
    "libpgo.so": ["pgo_kernels.hip", "pgo_capi.hip"],
}


def build(names=None, verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    built = []
    for name, srcs in LIBS.items():
        if names and name not in names:
            continue
        paths = [os.path.join(CSRC, s) for s in srcs]
        if not all(os.path.exists(p) for p in paths):
            continue
        out = os.path.join(HERE, name)
        cmd = [hipcc, *COMMON, "-I", os.path.join(os.path.dirname(HERE), "include"), "-o",
               out + ".tmp", *paths]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
        built.append(out)
    return built


if __name__ == "__main__":
    for p in build(sys.argv[1:] or None, verbose=True):
        print("built", p)
