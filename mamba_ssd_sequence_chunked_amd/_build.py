"""Build the HIP library (gfx950) in-tree: mamba_ssd_sequence_chunked_amd/libssd_mi355x.so.

Every .hip file under csrc/ is compiled by hipcc for gfx950 only and linked
into one shared library exporting the C ABI of include/ssd.h.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libssd_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off: hipcc would otherwise form v_pk_* from scalar float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fgpu-flush-denormals-to-zero",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every csrc/*.hip for gfx950 and link the shared library; returns its path."""
    objs = []
    with tempfile.TemporaryDirectory(prefix="ssd_build_") as tmp:
        procs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            while sum(p.poll() is None for _, p in procs) >= jobs:
                procs[[p.poll() is None for _, p in procs].index(True)][1].wait()
        failed = []
        for src, p in procs:
            out = p.communicate()[0].decode(errors="replace")
            lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                failed.append((src, "\n".join(lines)))
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            msg = "\n\n".join(f"{s}:\n{o}" for s, o in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = LIB_PATH + ".tmp"
        subprocess.check_call([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs])
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
