"""CPU sanitizer runs of the host-side code: the fp64 oracle's pins against an AddressSanitizer +
UndefinedBehaviorSanitizer build of oracle.c, and the host ABI checks against a build of the
library whose host code (abi.hip: every argument check) carries the same sanitizers. Each runs in
a child Python that preloads the matching ASan runtime (gcc's for the oracle, clang's for the
library), so a report of either sanitizer fails the child and this test. No GPU is used: the ABI
checks return before any launch."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TESTS = ["tests/test_oracle_formats.py", "tests/test_oracle_plan.py", "tests/test_oracle_gemm.py",
                "tests/test_oracle_route.py", "tests/test_oracle_mlp.py", "tests/test_oracle_fp8.py",
                "tests/test_oracle_shared.py"]


def _child(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter itself is not instrumented
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    from oracle import build
    lib = build.build(sanitize=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's ASan runtime is not installed")
    out = _child({"LD_PRELOAD": asan, "NVFP4_ORACLE_LIB": lib}, ORACLE_TESTS)
    assert " passed" in out


def test_host_abi_checks_under_asan_ubsan():
    from gemm_nvfp4_amd import build
    lib = build.build_host_sanitized()
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    out = _child({"LD_PRELOAD": rt[-1], "NVFP4_TEST_LIB": lib}, ["tests/test_abi_host.py"])
    assert " passed" in out
