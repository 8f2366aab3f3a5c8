"""Build libmla355.so (all HIP sources, gfx950 only) into this package directory.

Usage: python -m mla_decode_paged_02_amd.build [-v]
Every call compiles from scratch; objects go to a temporary folder.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla355.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


# Per-source extra flags.  The batch decode kernels keep their running scores in ordinary
# registers (the accumulation registers hold the output tile): their score MFMAs use the
# VGPR form.
EXTRA = {"mla_decode2.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "mla_fp8mma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, obj, verbose):
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(src)}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose=False):
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="mla355_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(srcs, objs)))
        tmp_lib = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
        os.replace(tmp_lib, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
