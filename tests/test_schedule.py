"""The attention kernel's work schedule on the CPU: tests/sched_coverage.cpp
builds the kernel's own scheduling header (host-only, with hipcc) and checks
that every work item is taken exactly once for a sweep of shapes and launch
sizes, and that in the XCD-grouped form each KV head's items stay on its XCDs."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_schedule_covers_every_item_once(tmp_path):
    exe = str(tmp_path / "sched_coverage")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "gated_gqa_causal_amd", "csrc"),
                    os.path.join(ROOT, "tests", "sched_coverage.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:]
    assert "schedule ok" in r.stdout
