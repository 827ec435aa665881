"""Compile libk3moe.so (the C-ABI library and its gfx950 kernels) in-tree."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libk3moe.so")
SOURCES = [os.path.join(CSRC, "k3moe_api.cpp"), os.path.join(CSRC, "k3moe_kernels.hip"),
           os.path.join(CSRC, "k3moe_grouped.hip"), os.path.join(CSRC, "k3moe_stream.hip"),
           os.path.join(CSRC, "k3moe_latent.hip"), os.path.join(CSRC, "k3moe_step.hip"),
           os.path.join(CSRC, "k3moe_cache.hip")]
HEADERS = [os.path.join(CSRC, "k3moe_internal.h"), os.path.join(ROOT, "include", "k3moe.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# gfx950 only; packed fp32 instructions disabled ("Build").
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-x", "hip"] + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("libk3moe build failed:\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
