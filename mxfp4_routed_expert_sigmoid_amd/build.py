"""Compile libk3moe.so (the C-ABI library and its gfx950 kernels) in-tree.

Each source compiles to its own object (in parallel; _build/ next to this
file), then one hipcc link makes the shared library."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libk3moe.so")
SOURCES = [os.path.join(CSRC, f) for f in (
    "k3moe_api.cpp", "k3moe_kernels.hip", "k3moe_decode.hip", "k3moe_grouped.hip", "k3moe_stream.hip",
    "k3moe_latent.hip", "k3moe_step.hip", "k3moe_cache.hip")]
HEADERS = [os.path.join(CSRC, "k3moe_internal.h"), os.path.join(CSRC, "k3moe_device.h"),
           os.path.join(ROOT, "include", "k3moe.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# gfx950 only; packed fp32 instructions disabled ("Build").
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-x", "hip", "-c", s, "-o", o] for s, o in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"libk3moe build failed ({os.path.basename(s)}):\n" + err)
        if verbose and err.strip():
            print(err)
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, err = _run(link)
    if rc != 0:
        raise RuntimeError("libk3moe link failed:\n" + err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
