"""Build libmk.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["mk_api.hip", "mk_layer.hip", "mk_aux.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 VALU forms (v_pk_fma/mul/add_f32) in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no unrolling of loops whose trip count is known only at run time.  It leaves the
    # specialised one-sequence layer kernel's code unchanged but shrinks the kernels emitted
    # before it, and the layer time depends on where that kernel's code sits in the code
    # object: measured 1.0 us per layer faster with this flag (the kernel at offset 0x69400)
    # than without it (0x68300), with identical code
    "-mllvm", "-unroll-runtime=false",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into layer_persistent_amd/libmk.so; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    extra = os.environ.get("MK_HIPCC_DEFINES", "").split()   # extra -D flags for experiments
    cmd = [HIPCC, *FLAGS, *extra, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
