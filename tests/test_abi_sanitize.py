"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

tmx_host.hip (validation, error strings, context bookkeeping) is compiled with
both sanitizers on its host code only, linked with the library's other
objects into tests/abi_sanitize_driver.c, and run on the CPU: every
validation path, the MXFP8 shape checks that once divided by H before
checking it, creation without a device, and every entry point with a NULL
context. Any sanitizer report (leaks included) fails the run."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def test_host_abi_under_asan_ubsan(tmp_path):
    for tool in (HIPCC, CLANG, CLANGXX):
        if not os.path.exists(tool):
            pytest.skip(f"{tool} not available")
    import torch
    if torch.cuda.is_available():
        pytest.skip("runs the no-device paths; a GPU is present")
    from token_moe_amd import build as b
    objs = [os.path.join(b.OBJ, src.replace(".hip", ".o")) for src in b.SOURCES if src != "tmx_host.hip"]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    host_o = str(tmp_path / "tmx_host_asan.o")
    # sanitizers on the host code only (each flag behind -Xarch_host)
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([HIPCC, *flags, *san, "-c", os.path.join(b.CSRC, "tmx_host.hip"), "-o", host_o],
                   check=True, capture_output=True)
    drv_o = str(tmp_path / "driver.o")
    subprocess.run([CLANG, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.c"),
                    "-o", drv_o], check=True, capture_output=True)
    exe = str(tmp_path / "driver")
    subprocess.run([CLANGXX, "-fsanitize=address,undefined", "-o", exe, drv_o, host_o, *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi-sanitize ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
