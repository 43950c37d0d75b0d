"""The two-piece key-limit form that the dK/dV kernel evaluates per tile on the scalar unit
(make_kv_form / kv_form_eval) agrees with kv_limit, the per-row rule every kernel uses,
for every layout, shard pair and row of small shapes and at the edge rows of L = 2^20.
Compiled from tests/kv_form_check.cpp against the library's internal header; host only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_kv_form_matches_kv_limit(tmp_path):
    exe = tmp_path / "kv_form_check"
    cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "ring_attention_long_amd", "csrc"),
           os.path.join(ROOT, "tests", "kv_form_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], check=False, capture_output=True, text=True, timeout=120)
    n, bad = map(int, out.stdout.split())
    assert n > 200000
    assert bad == 0 and out.returncode == 0
