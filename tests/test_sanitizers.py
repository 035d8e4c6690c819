"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code (no GPU):

  * the CPU oracle (oracle/moe_oracle.c), every function driven on small
    inputs by tests/sanitize/oracle_driver.c;
  * the C ABI's host side (every argument check, the size queries including
    sizes that would overflow, the status strings), with the library built
    for gfx950 with sanitizers on its host code only, driven by
    tests/sanitize/capi_driver.c.
Any out-of-range access, signed overflow or other undefined behaviour aborts
the driver (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-o", exe,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "clean" in r.stdout


def test_c_abi_host_side_under_asan_ubsan(tmp_path):
    hipcc, clang = "/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    from sigmoid_top_routing_02_amd import build as b
    lib = str(tmp_path / "libmoefp8_san.so")
    # the product flags with the device code still at -O3 (its inline asm
    # needs operands the optimiser proves wave-uniform), the host code at -O1
    # with the sanitizers
    flags = [f for f in b.FLAGS if f not in ("-O3", "-Wall")] + ["-Xarch_device", "-O3"]
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    _run([hipcc, *flags, *host_san, "-I", os.path.join(ROOT, "include"), "-o", lib, *b.sources()])
    exe = str(tmp_path / "capi_driver")
    _run([clang, *SAN, "-I", os.path.join(ROOT, "include"), "-o", exe, os.path.join(HERE, "capi_driver.c"), lib,
          f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=ENV)
    assert "clean" in r.stdout and "runtime error" not in r.stderr
