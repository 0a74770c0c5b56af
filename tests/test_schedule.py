"""The plans of csrc/internal.h, on the CPU: the tiled gate/up kernel's
item <-> workgroup maps are exact inverses, leave no item out and none
twice, stay inside the launch and the workspace for every plan, and keep the
eight XCDs' shares within one last-round share; the few-token plans route in
the gate/up kernel's prologue only within its limits and choose whole tile
columns only where that kernel's loads hold (host build of
tests/sched/sched_check.cpp, with UBSan on the host pass)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_schedule_maps(tmp_path):
    exe = str(tmp_path / "sched_check")
    r = subprocess.run([HIPCC, "-O1", "-std=c++17", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all",
                        os.path.join(ROOT, "tests", "sched", "sched_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.stdout[-2000:], r.stderr[-2000:])
    assert "runtime error" not in r.stderr, r.stderr[-2000:]
