"""Host code under AddressSanitizer and UBSan (CPU only).

* The C ABI's host side: tests/sanitize_abi.cpp calls every refusal path of
  the validation, the batch planner, the size queries and the null-context
  entry points.  The library's sources are built with hipcc, sanitizers on the
  host code only (each -fsanitize after -Xarch_host); no device is touched.
* The CPU oracle: tests/sanitize_oracle.c compiles oracle.c into a driver
  (gcc) that runs every entry point on edge shapes with exact-size buffers.
"""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    print(r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_abi_host_side_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "gated_gqa_causal_amd", "csrc")
    exe = str(tmp_path / "sanitize_abi")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "abi.cpp"), os.path.join(csrc, "kernels.hip"),
           os.path.join(ROOT, "tests", "sanitize_abi.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    r = _run(exe)
    assert r.returncode == 0 and "abi host checks ok" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_oracle")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-o", exe,
                    "-lm"], check=True, capture_output=True)
    r = _run(exe)
    assert r.returncode == 0 and "oracle checks ok" in r.stdout
