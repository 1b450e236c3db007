"""The single-launch step's work protocol on the host (no GPU needed).

tests/step_protocol_host.cpp runs the kernel's protocol code (run_step_protocol
of qk_norm_rope_amd/csrc/step_protocol.h) over the same control-word layout,
with one host thread per workgroup and fewer resident workgroups than the grid:
tickets, publication, the bounded wait, phase 2 and the exit that leaves the
words zero. Planting a mistake in the protocol (no wait, the first workgroup out
clearing the words, an off-by-one ticket bound) makes it fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "step_protocol_host.cpp")
BIN = os.path.join(ROOT, "_build", "step_protocol_host")


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        pytest.skip("hipcc not found")
    return path


def test_step_protocol_on_host_threads():
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    cmd = [_hipcc(), "-x", "hip", "--cuda-host-only", "-std=c++17", "-O2", "-pthread", "-Wall",
           "-I", os.path.join(ROOT, "qk_norm_rope_amd", "csrc"), SRC, "-o", BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=180)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 failed" in r.stdout
