"""Build the HIP library libdecode_attn.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libdecode_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 (v_pk_*_f32) code generation is disabled on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ into one shared library (always rebuilds)."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed building %s" % LIB_NAME)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
