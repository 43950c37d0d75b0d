"""The split plans of batched forward launches (plan_split_batch): items map one to one onto
query blocks, launch in nonincreasing cost, at most 128 of them; splits where idle units or an
imbalanced full grid gain, none for equal blocks that fill the units, none with packed
documents; the cached plan equals the computed one.  Compiled from tests/batch_plan_check.cpp
against the library's internal header and linked with libra.so; host only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
LIBDIR = os.path.join(ROOT, "ring_attention_long_amd")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.skipif(not os.path.exists(os.path.join(LIBDIR, "libra.so")), reason="libra.so not built")
def test_batch_split_plans(tmp_path):
    exe = tmp_path / "batch_plan_check"
    cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(LIBDIR, "csrc"),
           os.path.join(ROOT, "tests", "batch_plan_check.cpp"), "-L", LIBDIR, "-lra",
           f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    out = subprocess.run([str(exe)], check=False, capture_output=True, text=True, timeout=120, env=env)
    n, bad = map(int, out.stdout.split())
    assert n > 1000, out.stderr[-2000:]
    assert bad == 0 and out.returncode == 0, out.stderr[-2000:]
