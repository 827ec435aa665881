"""The oracle and the C ABI's host-side validation built with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU (the
kimi-k3-in-c README, Part I "Common questions", ships asan and ubsan builds
of its C). Each driver under tests/sanitize/ exits 0 and prints "ok" only
when every call returned what its contract says; any sanitizer report
aborts the run (no recovery).

The library's host code is compiled with the sanitizers on the host side
only (its gfx950 device code is built as usual) and linked with the kernel
objects of the normal build; only paths that return before the first HIP
runtime call are driven, so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_GCC = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-static-libasan", "-static-libubsan"]
# host-side only: each sanitizer flag is preceded by -Xarch_host
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    r.stderr = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r


def _gcc(tmp, name, sources):
    exe = os.path.join(tmp, name)
    r = _run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-ffp-contract=off"] + SAN_GCC +
             ["-o", exe] + sources + ["-lm"])
    assert r.returncode == 0, r.stderr
    return exe


def _clean_run(exe):
    r = _run([exe], timeout=300, env=dict(os.environ, OMP_NUM_THREADS="4"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok", r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr


@pytest.fixture
def tmp(tmp_path):
    return str(tmp_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp):
    exe = _gcc(tmp, "oracle_asan", [os.path.join(HERE, "oracle_driver.c"),
                                     os.path.join(ROOT, "oracle", "k3moe_oracle.c")])
    _clean_run(exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_sanitized_build_reports_an_overrun(tmp):
    # the same flags catch a read one element past a heap buffer (UBSan's
    # object-size check or ASan, whichever sees it first)
    src = os.path.join(tmp, "overrun.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\nint main(int c, char **v) { (void)v;\n"
                "  int *p = malloc(4 * sizeof(int)); for (int i = 0; i < 4; i++) p[i] = i;\n"
                "  int s = p[c + 3]; free(p); return s; }\n")
    exe = _gcc(tmp, "overrun", [src])
    r = _run([exe], timeout=60)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr, r.stderr


def _library_objects():
    obj = os.path.join(ROOT, "mxfp4_routed_expert_sigmoid_amd", "_build")
    names = ["k3moe_kernels.hip.o", "k3moe_decode.hip.o", "k3moe_grouped.hip.o", "k3moe_stream.hip.o",
             "k3moe_latent.hip.o", "k3moe_step.hip.o", "k3moe_cache.hip.o"]
    paths = [os.path.join(obj, n) for n in names]
    return paths if all(os.path.exists(p) for p in paths) else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_api_host_validation_under_asan_and_ubsan(tmp):
    objs = _library_objects()
    if objs is None:
        pytest.skip("library objects not built (run __graft_entry__.build())")
    inc = ["-I", os.path.join(ROOT, "include")]
    api_o, drv_o, exe = (os.path.join(tmp, n) for n in ("api.o", "driver.o", "api_asan"))
    src = os.path.join(ROOT, "mxfp4_routed_expert_sigmoid_amd", "csrc", "k3moe_api.cpp")
    r = _run([HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops"] + SAN_HOST + inc + ["-x", "hip", "-c", src, "-o", api_o])
    assert r.returncode == 0, r.stderr
    r = _run([HIPCC, "-O1", "-g", "-std=c++17", "-x", "c++"] + SAN_HOST + inc +
             ["-c", os.path.join(HERE, "api_driver.cpp"), "-o", drv_o])
    assert r.returncode == 0, r.stderr
    r = _run([HIPCC, "--offload-arch=gfx950"] + SAN_HOST + [drv_o, api_o] + objs + ["-o", exe])
    assert r.returncode == 0, r.stderr
    _clean_run(exe)
