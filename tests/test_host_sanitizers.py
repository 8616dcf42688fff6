"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer:

* the fp64 oracle (plain C), driven through every entry point on small
  problems whose buffers are exactly sized (tests/sanitize/oracle_driver.c);
* the host side of the C ABI (descriptor validation, plans, the tile
  schedule, workspace sizing, the run-time argument checks), with the kernel
  launchers stubbed out (tests/sanitize/api_driver.cpp).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "swa_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAILED" not in r.stdout and r.stdout.count(" ok") == 3, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_c_abi_host_side_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    csrc = os.path.join(ROOT, "sliding_window_attention_flash_amd", "csrc")
    # host-only sanitizers: each -fsanitize= applies to the host pass
    cmd = [HIPCC, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "api driver: ok" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
