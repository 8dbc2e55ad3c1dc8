"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host code (packers, the C ABI, the host side of the kernel
files) and the oracle are rebuilt with ASan + UBSan (build_sanitized in
sparse_dense_matrix_amd/build.py and oracle/__init__.py), then
  - tests/sanitize_driver.c walks every packer through forced allocation
    failures (SPMM_TEST_FAIL_ALLOC) and exits under the leak detector: no
    block may be left behind by a failing or a successful pack;
  - the rest of the CPU suite (-m "not gpu") runs against the sanitized
    builds in a child process that preloads the ASan runtime (leak detection
    off there: the interpreter itself is not leak-clean).
Any report aborts the child and fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.fixture(scope="module")
def sanitized():
    if not os.path.exists(CLANG):
        pytest.skip("clang of the ROCm toolchain not found")
    sys.path.insert(0, os.path.join(ROOT, "sparse_dense_matrix_amd"))
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "sdm_build", os.path.join(ROOT, "sparse_dense_matrix_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    import oracle
    return {"lib": b.build_sanitized(), "oracle": oracle.build_sanitized(),
            "runtime": b.asan_runtime()}


def test_packer_failure_paths_leak_nothing(sanitized, tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    lib = sanitized["lib"]
    subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize_driver.c"), "-o", exe, lib,
                    f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("SPMM_TEST_FAIL_ALLOC", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-3000:], r.stderr[-6000:])
    assert r.returncode == 0 and "driver ok" in r.stdout


def test_cpu_suite_under_asan_ubsan(sanitized):
    env = dict(os.environ, LD_PRELOAD=sanitized["runtime"],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               SPMM_LIBRARY=sanitized["lib"], ORACLE_LIBRARY=sanitized["oracle"])
    env.pop("SPMM_TEST_FAIL_ALLOC", None)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider",
                        "--ignore", os.path.join(ROOT, "tests", "test_sanitizers.py")],
                       capture_output=True, text=True, env=env, timeout=1200, cwd=ROOT)
    print(r.stdout[-3000:], r.stderr[-6000:])
    assert r.returncode == 0, "sanitized CPU suite failed"
    assert "passed" in r.stdout
