"""The oracle and the C ABI's host-side validation, built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven over their edge cases (CPU only; the drivers are in
tests/sanitize/). Any report, leak aside, fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-3000:]}\n{p.stderr[-3000:]}"
    return p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = os.path.join(str(tmp_path), "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    assert "oracle driver: ok" in run([exe], env=ENV, timeout=600)


def test_abi_validation_under_sanitizers(tmp_path):
    from calibration_free_weight_amd import build as hb
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    objdir = os.path.join(hb.PKG, "_build")
    others = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in hb.sources()
              if not s.endswith("hqq_api.hip")]
    if not all(os.path.exists(o) for o in others):
        hb.build(stress=False)
    d = str(tmp_path)
    api_o = os.path.join(d, "hqq_api_san.o")
    # host code instrumented, device code built as usual
    san = ["-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    run([hipcc, *hb.HIPCC_FLAGS, *san, "-g", "-c", "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(hb.PKG, "csrc"), "-o", api_o,
         os.path.join(hb.PKG, "csrc", "hqq_api.hip")])
    drv_o = os.path.join(d, "abi_driver.o")
    run([hipcc, "-O1", "-g", "-std=c++17",
         "-fsanitize=address", "-fsanitize=undefined",
         "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
         os.path.join(SAN, "abi_driver.cpp"), "-o", drv_o])
    exe = os.path.join(d, "abi_driver")
    run([hipcc, f"--offload-arch={hb.ARCH}",
         "-fsanitize=address", "-fsanitize=undefined",
         "-o", exe, drv_o, api_o, *others])
    assert "abi driver: ok" in run([exe], env=ENV, timeout=600)
