"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the library's
sources are compiled with both sanitizers on the host side only (device code unchanged) and
linked into tests/abi_sanitize.cpp, which calls every entry point with arguments that
validation must refuse (no device is touched) and runs the host-only helpers on valid inputs.
Any sanitizer report aborts the program; any wrong status is counted."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.timeout(900)
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    from ring_attention_long_amd import build as B

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        r = subprocess.run([HIPCC, *B.FLAGS, *SAN_HOST, "-g", "-c", src, "-o", obj], capture_output=True,
                           text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, B.sources()))
    drv = str(tmp_path / "driver.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    subprocess.run([CLANG, "-O1", "-g", *san, "-std=c++17", "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-o", drv], check=True, timeout=300)
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([CLANG, *san, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", exe], check=True, timeout=300)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0, out.stdout + out.stderr[-4000:]
    n, bad = map(int, out.stdout.split())
    assert n > 150 and bad == 0
