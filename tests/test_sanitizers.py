"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two builds, made here with the host compilers (no GPU code is involved):
- the C-ABI layer (conv3d_api.cpp: checks, planning, workspace carving,
  dispatch) linked with host stand-ins for the kernel launchers, driven
  through every entry point with valid and rejected calls
  (tests/sanitize/api_driver.cpp);
- the C oracle on small shapes with every post-operation flag and pixel
  lists, each output sized exactly (tests/sanitize/oracle_driver.c).
Any out-of-range access, overflow or other undefined behaviour aborts the
driver and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")


def _build_and_run(tmp_path, compiler, srcs, extra, out, expect):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / out)
    cmd = [compiler, *extra, *SAN, *[os.path.join(ROOT, s) for s in srcs], "-o", exe]
    if compiler == "gcc":
        cmd.append("-lm")
    subprocess.run(cmd, check=True, cwd=str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600,
                       cwd=str(tmp_path))
    assert r.returncode == 0, r.stdout + r.stderr
    assert expect in r.stdout


def test_c_abi_layer_under_sanitizers(tmp_path):
    _build_and_run(tmp_path, "g++",
                   ["tests/sanitize/api_driver.cpp", "tests/sanitize/stub_launchers.cpp",
                    "convolution_video_vae_amd/csrc/conv3d_api.cpp"],
                   ["-std=c++17", "-Wall"], "api_driver", "api driver ok")


def test_oracle_under_sanitizers(tmp_path):
    _build_and_run(tmp_path, "gcc",
                   ["tests/sanitize/oracle_driver.c", "oracle/conv3d_oracle.c"],
                   ["-std=c11", "-fopenmp", "-ffp-contract=off", "-Wall"], "oracle_driver",
                   "oracle driver ok")
