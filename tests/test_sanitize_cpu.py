"""Memory and undefined-behaviour checks of the host code, on the CPU.

The plain-C oracle and the HIP library's host side (blob sizes, the host
repack at every weight format, validation, the allocation cap) are built
with AddressSanitizer and UndefinedBehaviorSanitizer and driven by the small
programs under tests/sanitize/.  Device code is built without sanitizers
(there is no GPU here); the drivers call nothing that launches a kernel.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "int4_routed_expert_layer_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout + r.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         os.path.join(ROOT, "oracle", "coli_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
         "-o", exe, "-lm"])
    out = run([exe], env=SAN_ENV)
    assert "oracle driver ok" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    # Host code sanitized, device code not (each -fsanitize= applies to the
    # host side only).
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        procs.append((subprocess.Popen([HIPCC, *flags, *host_san, "-c", src, "-o", obj],
                                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    for p, src in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{src}\n{out}\n{err}"
    drv_obj = str(tmp_path / "abi_driver.o")
    gxx = shutil.which("g++") or "g++"
    run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv_obj])
    exe = str(tmp_path / "abi_driver")
    run([HIPCC, "--offload-arch=gfx950", *host_san, drv_obj, *objs, "-o", exe])
    # Leak checking stays off here: the HIP runtime's own start-up
    # allocations are not this library's.
    env = dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0")
    out = run([exe], env=env)
    assert "abi driver ok" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out
