"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

The oracle (plain C) and the library's host code (validation, constants,
workspace sizes, shadow-region headers, argument checks) are built with
both sanitizers -- for the library on the host side only, its device code
built as usual and never launched -- and driven by small programs under
tests/sanitize/ that call every host-side entry point on exactly-sized
inputs, edge sizes and error paths.  A read or write past an array, a use
after free, a leak or an undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "layer_streamed_optimizer_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-pthread", os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "adam_oracle.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    assert "all calls returned their documented codes" in run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_runtime_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "runtime_driver")
    from layer_streamed_optimizer_amd import build
    srcs = [os.path.join(CSRC, f) for f in build.LIBS["liblso.so"]]   # the library's own source list
    # each sanitizer flag applies to the host pass only
    host_san = ["-Xarch_host", "-fsanitize=address",
                "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(HERE, "runtime_driver.cpp"), *srcs, "-o", exe, "-lhsa-runtime64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "every call returned its documented status" in run(exe)
