"""The host side of the C ABI and the fp64 oracle, built with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

The ABI's host layer (gdn_tree_api.cpp) is linked against stand-ins for the
three HIP runtime calls it makes and for the kernel launchers
(tests/sanitize/host_stubs.cpp), with host memory standing in for device
memory, so every argument check, the context, the GDN_VALIDATE host checks
and the status read-back run under the sanitizers.  The oracle is driven on
small seeded trees (tests/sanitize/oracle_driver.c).  Both are plain g++/gcc
builds of host code only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_deltanet_tree_gdn_amd", "csrc")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_abi_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    _build(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", SAN,
            os.path.join(CSRC, "gdn_tree_api.cpp"), os.path.join(SAN, "host_stubs.cpp"),
            os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    _run(exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c99", *FLAGS, "-ffp-contract=off", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
            os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm", "-lpthread"])
    _run(exe)
