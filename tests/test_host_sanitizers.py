"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the C oracle (oracle/mxfp8_oracle.c) and the C-ABI layer of the library (abi.cpp and
paths.cpp, with host stubs for the HIP launchers: tests/sanitize/launch_stubs.cpp) with g++ /
gcc ``-fsanitize=address,undefined``, then runs the ABI contract suite (test_abi_cpu.py) and
the oracle-pin suite (test_oracle_pins.py) against those builds in a child interpreter with
the ASan runtime preloaded.  Any sanitizer report aborts the child, so the suites must pass
clean.  No GPU code is built or run here."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_partial_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs the host C/C++ compilers")


def runtime(name):
    path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitized")
    abi = str(d / "libmxfp8partial_san.so")
    orc = str(d / "libmxfp8_oracle_san.so")
    from mxfp8_block_scaled_partial_amd import build as hip_build

    subprocess.check_call(
        ["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
         f'-DMXFP8_KERNEL_SOURCE_HASH="{hip_build.kernel_source_hash()}"',
         "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{CSRC}",
         os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "paths.cpp"),
         os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", abi])
    subprocess.check_call(
        ["gcc", "-std=c11", "-fPIC", "-shared", *SAN, "-fno-fast-math", "-ffp-contract=off",
         os.path.join(ROOT, "oracle", "mxfp8_oracle.c"), "-lm", "-o", orc])
    return abi, orc


def test_abi_and_oracle_suites_pass_under_asan_and_ubsan(sanitized):
    abi, orc = sanitized
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's libasan.so is not installed")
    env = dict(os.environ, LD_PRELOAD=asan, MXFP8_PARTIAL_LIB=abi, MXFP8_ORACLE_LIB=orc,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         os.path.join(ROOT, "tests", "test_abi_cpu.py"),
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    # the children really loaded the sanitized builds
    assert " passed" in r.stdout


def test_sanitized_builds_are_the_ones_the_suites_load(sanitized):
    """The binding and the oracle wrapper pick up the builds named in the environment."""
    abi, orc = sanitized
    code = ("from mxfp8_block_scaled_partial_amd import binding as B; import oracle; "
            "print(B.LIB_PATH); print(oracle._LIB)")
    env = dict(os.environ, MXFP8_PARTIAL_LIB=abi, MXFP8_ORACLE_LIB=orc)
    out = subprocess.check_output([sys.executable, "-c", code], cwd=ROOT, env=env, text=True)
    assert out.split() == [abi, orc]
