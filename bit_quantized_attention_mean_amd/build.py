"""Builds libsage_attn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel),
then linked into bit_quantized_attention_mean_amd/libsage_attn.so. The library
is replaced atomically, so a failed build leaves the previous one in place.
Run: python bit_quantized_attention_mean_amd/build.py (by path: importing it
through the package would first load the library it is about to build).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsage_attn.so")
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that note is harmless.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def check_kernel_stubs(objs) -> None:
    """Every kernel a launcher references must be defined in its object. The host
    pass of hipcc can drop a kernel template instantiation without a diagnostic
    (its host stub then stays undefined and the library would lack the kernel),
    so an undefined __device_stub__ symbol fails the build."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    for o in objs:
        r = subprocess.run([nm, o], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{nm} {o} failed:\n{r.stdout}")
        missing = [l.split()[-1] for l in r.stdout.splitlines()
                   if "__device_stub__" in l and l.split()[-2:-1] == ["U"]]
        if missing:
            raise RuntimeError(f"{os.path.basename(o)}: kernel(s) dropped by the host pass: {missing[:4]}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda so: _run([cc, *HIP_FLAGS, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    if verbose:
        for o in outs:
            if o:
                print(o)
    check_kernel_stubs(objs)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
