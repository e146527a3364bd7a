"""Builds libmsa.so (all HIP sources for gfx950) in the package directory."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsa.so")
LIB_SAN = os.path.join(PKG, "libmsa_san.so")
SOURCES = ["abi.cpp", "pool.hip", "route.hip", "topk.hip", "gather.hip", "decode.hip", "prefill.hip", "encode.hip"]
ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden", "--offload-arch=" + ARCH,
         # packed fp32 VALU forms are kept out of generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA accumulators in VGPRs: the AGPR form makes the register allocator copy
         # accumulators between the two files on every loop iteration
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (each -fsanitize= applies to the host pass
# only; the device code is built as usual).  For CPU-only runs of the host checks.
SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, src + (".san.o" if sanitize else ".o"))
    cmd = ["hipcc", "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + FLAGS + (SAN_FLAGS if sanitize else [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Builds libmsa.so; with sanitize=True libmsa_san.so, whose host code is instrumented."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    lib_path = LIB_SAN if sanitize else LIB
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, lib_path)
    if verbose:
        print("built", lib_path)
    return lib_path


if __name__ == "__main__":
    build(verbose=True)
