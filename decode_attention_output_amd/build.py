"""Build the HIP library libdecode_attn.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled to its own object in parallel (each
holds its kernels and all device code they call), then linked once."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libdecode_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 (v_pk_*_f32) code generation is disabled on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _quiet(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return res.returncode, _quiet(res.stdout)


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ and link the shared library (always rebuilds)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC] + FLAGS + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if out.strip() and (rc != 0 or verbose):
            sys.stderr.write(out + "\n")
        failed |= rc != 0
    if failed:
        raise RuntimeError("hipcc failed building %s" % LIB_NAME)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    rc, out = _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp])
    if rc != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed linking %s" % LIB_NAME)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
