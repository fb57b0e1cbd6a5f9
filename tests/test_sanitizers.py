"""The oracle and libflarepp's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/sanitize/oracle_driver.c runs every oracle entry point (all dtypes,
shared and per-head seeds, edge shapes, argument errors);
tests/sanitize/host_driver.cpp runs the library's descriptor, tuning,
workspace and pointer validation for every call, each failing before any HIP
call (no GPU needed).  Both are built with the sanitizers (host code only:
on the hipcc line every -fsanitize= follows -Xarch_host; the device code of
the library is compiled as usual and never runs) and must exit cleanly."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)} -> {res.returncode}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-Wall", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "flarepp_oracle.c"), "-lm"])
    res = run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "all checks passed" in res.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
         "-Xarch_host", "-g",
         "-Xarch_host", "-fsanitize=address",
         "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-Xarch_host", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "rank_latent_attention_seed_amd", "csrc"),
         "-o", exe, os.path.join(ROOT, "rank_latent_attention_seed_amd", "csrc", "flarepp.hip"),
         os.path.join(HERE, "host_driver.cpp")], timeout=600)
    # the HIP runtime keeps allocations until exit: leak checking is for the oracle driver
    res = run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert "all checks passed" in res.stdout
