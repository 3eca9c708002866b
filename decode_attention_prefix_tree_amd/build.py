"""Build libchunkattn.so in-tree with hipcc for gfx950.

    python -m decode_attention_prefix_tree_amd.build

The host parts (manager, C-ABI) and the kernels go into one shared library.
HIP code is compiled without packed-fp32 instructions (the
``-packed-fp32-ops`` target feature is switched off) and without implicit
FMA contraction (``-ffp-contract=off``): fused multiply-adds appear only where
the source calls fmaf, so every instantiation of a kernel rounds the same way
and the one-launch and two-launch steps agree bit for bit.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libchunkattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HOST_SOURCES = ["manager.cpp", "capi.cpp"]
HIP_SOURCES = ["kernels.hip", "kv_write.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}", "-I/opt/rocm/include"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-ffp-contract=off"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    # hipcc's host pass does not know the packed-fp32 feature; drop that warning
    noise = [ln for ln in (r.stdout + r.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if verbose and noise:
        print("\n".join(noise))


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="chunkattn_build_") as tmp:
        objs = []
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, "-x", "c++", *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj],
                 verbose)
            objs.append(obj)
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src + ".o")
            _run([cc, "-x", "hip", *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([cc, *HIP_FLAGS, "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        # atomic replace, so a process that has the old library mapped keeps it
        dst_tmp = LIB_PATH + ".tmp"
        shutil.copyfile(tmp_lib, dst_tmp)
        os.replace(dst_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
