"""Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The C-ABI layer (hybrid_linear_attention_gated_amd/csrc/gdn_api.cpp: argument
  validation, overlap checks, workspace layout, the debug check and the status query) is
  built with g++ against host stand-ins for the kernel launchers (tests/sanitize/
  stub_launchers.cpp) and driven through every entry point, valid and invalid arguments
  (tests/sanitize/api_driver.cpp), once plainly and once with GDN_DEBUG_CHECK=1.
* The fp64 oracle (oracle/gdn_oracle.c) is built with gcc and run on small varlen inputs
  (tests/sanitize/oracle_driver.c).

Any sanitizer report aborts the program (-fno-sanitize-recover=all), failing the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _have(tool):
    return shutil.which(tool) is not None


def _build(cmd, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    if r.returncode != 0 and ("cannot find -lasan" in r.stderr or "libasan" in r.stderr):
        pytest.skip("no sanitizer runtime for this compiler")
    assert r.returncode == 0, r.stderr[-3000:]


@pytest.mark.skipif(not (_have("g++") and os.path.isdir("/opt/rocm/include")), reason="g++ / HIP headers")
def test_api_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_driver")
    csrc = os.path.join(ROOT, "hybrid_linear_attention_gated_amd", "csrc")
    _build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
            os.path.join(csrc, "gdn_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", exe], tmp_path)
    for debug in ("0", "1"):
        r = subprocess.run([exe], capture_output=True, text=True, env=dict(ENV, GDN_DEBUG_CHECK=debug), timeout=120)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "api driver ok" in r.stdout
        assert ("debug checks exercised" in r.stdout) == (debug == "1")


@pytest.mark.skipif(not _have("gcc"), reason="gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c99", *SAN, "-fno-fast-math", "-ffp-contract=off", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
            os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "oracle driver ok" in r.stdout
