"""Sanitizer builds of host code (CPU only).

The C ABI layer's argument validation (gdr_api.cpp) and the fp64 oracle are
compiled with AddressSanitizer and UndefinedBehaviorSanitizer (host code
only, with g++ / gcc) into small drivers under tests/sanitize/, which call
them with swept and edge-case arguments; a report from either sanitizer, a
crash or a failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    rc, out = _run(["gcc", "-std=c99", *SAN, "-fopenmp", os.path.join(HERE, "oracle_check.c"),
                    os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-lm", "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    rc, out = _run([exe], env=env)
    print(out)
    assert rc == 0 and out.startswith("ok"), out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_abi_validation_under_asan_ubsan(tmp_path):
    pkg = os.path.join(ROOT, "gated_delta_rule_24_amd")
    lib = os.path.join(pkg, "libgdr.so")
    if not os.path.exists(lib):
        pytest.skip("libgdr.so not built")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "abi_check")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_check.cpp"),
                    os.path.join(pkg, "csrc", "gdr_api.cpp"), "-L", pkg, "-lgdr", "-Wl,-rpath," + pkg,
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"),
                    "-o", exe])
    assert rc == 0, out
    # the HIP runtime keeps allocations until exit; leaks are not what is checked here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, out = _run([exe], env=env)
    print(out)
    assert rc == 0 and (out.startswith("ok") or out.startswith("skipped")), out
