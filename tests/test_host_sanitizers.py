"""Host-side sanitizers (CPU, no GPU): the library's host code -- argument
validation, workspace planning, the status and error strings -- built with
AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged), and
the C-ABI tests of test_abi_cpu.py plus a sweep of extreme descriptors run
against that build in a child process with the sanitizer runtime preloaded.
Any report aborts the child and fails the test."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_token_verification_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) or not ASAN_RT,
                                reason="hipcc or the sanitizer runtime is not installed")

SWEEP = r'''
import ctypes, itertools, sys
sys.path.insert(0, sys.argv[1])
import lossless_token_verification_amd as sv
lib = sv.library()
vals32 = [-2**31, -1, 0, 1, 7, 63, 64, 4096, 1 << 20, (1 << 20) + 1, 2**31 - 1]
n = 0
for B, k, V, dt in itertools.product(vals32, [-1, 0, 1, 8, 63, 64, 2**31 - 1],
                                     [-1, 0, 1, 128256, 1 << 20, 2**31 - 1], [0, 1, 2, -1]):
    for ld in (0, 1, 2**40, 2**62):
        d = sv.make_desc(B, k, V, dt, ld)
        for exits in (2, 3, 4):
            lib.spec_verify_workspace_bytes(ctypes.byref(d), exits)
            lib.spec_verify_validate(ctypes.byref(d), exits, 4, 1 << 30)
        lib.spec_verify_lmhead_workspace_bytes(ctypes.byref(d), 4096)
        lib.spec_verify_lmhead_workspace_bytes(ctypes.byref(d), -64)
        lib.spec_verify_tentative_workspace_bytes(ctypes.byref(d), 9)
        lib.spec_verify_tentative_workspace_bytes(ctypes.byref(d), 2**31 - 1)
        n += 1
for code in range(-3, 10):
    lib.spec_verify_status_string(code)
lib.spec_verify_last_error()
print("sweep", n)
'''


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asan") / "libspecverify.so")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *srcs, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-3000:]
    return out


def _env(lib):
    env = dict(os.environ)
    env["SPEC_VERIFY_LIB"] = lib
    env["LD_PRELOAD"] = ASAN_RT[-1]
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def test_abi_tests_under_host_sanitizers(asan_lib):
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=_env(asan_lib), capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr


def test_extreme_descriptors_under_host_sanitizers(asan_lib):
    res = subprocess.run([sys.executable, "-c", SWEEP, ROOT], cwd=ROOT, env=_env(asan_lib),
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert "sweep" in res.stdout and "runtime error" not in res.stderr
