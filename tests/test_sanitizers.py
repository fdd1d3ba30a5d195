"""AddressSanitizer and UBSan over the host code, on the CPU.

Two host-only builds with both sanitizers, in a temporary directory:
 - the fp64 oracle (oracle/oracle.c), driven by every oracle pin;
 - the C-ABI validation layer (sparse_paged_mla_amd/csrc/api.cpp) with its
   kernel launchers replaced by counting stubs (tests/sanitize), driven by
   the boundary tests, including calls that pass validation.
Both run in a child interpreter with the ASan runtime preloaded; any
sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc's ASan runtime is not installed")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    oracle_lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
                    "-o", oracle_lib, "-lm"], check=True)
    csrc = os.path.join(ROOT, "sparse_paged_mla_amd", "csrc")
    api_lib = str(tmp_path / "libsparse_mla_validate_asan.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
                    "-o", api_lib, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", SPMLA_ORACLE_LIB=oracle_lib,
               SPMLA_BOUNDARY_LIB=api_lib, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]
    # The child really used the sanitizer builds.
    probe = ("import ctypes, oracle, os; oracle._load(); import tests.test_boundary as tb; "
             "print(oracle._LIB_PATH == os.environ['SPMLA_ORACLE_LIB'], tb.STUB_LIB == os.environ['SPMLA_BOUNDARY_LIB'])")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.stdout.split() == ["True", "True"], r.stdout + r.stderr
