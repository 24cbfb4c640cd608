"""Build libduo.so (host C ABI + HIP kernels for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libduo.so")
ARCH = "gfx950"
SOURCES = ["duo_host.cpp", "duo_kernels.hip", "duo_prefill.hip", "duo_gated.hip"]

# Packed fp32 VALU ops are turned off for device code (the host pass warns that
# it does not know the feature; that is expected).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Per-source device flags.  The prefill and gated kernels' MFMA results (scores and the
# output accumulators) are read by the softmax and the final scaling on the
# vector ALU; asking for the VGPR form of MFMA keeps them out of the
# accumulation registers, which saves a read-out and a zero fill per tile.
SOURCE_FLAGS = {"duo_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "duo_gated.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = True, jobs: int = 4) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        path = os.path.join(CSRC, src)
        if src.endswith(".hip"):
            cmd = [cc, f"--offload-arch={ARCH}", "-x", "hip", *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []),
                   "-c", path, "-o", obj]
        else:
            cmd = [cc, *COMMON, "-c", path, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(ln for ln in text.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{text}")
        if verbose and text.strip():
            print(text, file=sys.stderr)
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (say, a kernel whose host stub the compiler
    # dropped) fails the link instead of the first load
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stdout.decode(errors='replace')}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
