"""Host sanitizer run (CPU only): the fp64 oracle (oracle/oracle.c) and the
C ABI (abi.cpp, plan.cpp) compiled with -fsanitize=address,undefined, the
ABI linked against a test double of the kernel launchers that records each
launch instead of running it (tests/host_double/recorder.cpp).  A child
pytest process then runs the oracle's pins and the ABI tests against those
builds, plus the recorded-launch tests of tests/host_double/; any sanitizer
report, and any launch that breaks the launchers' stated argument
invariants, fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "megatron_tensor_transformer_colpar_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    if runtime("libasan.so") is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    d = tmp_path_factory.mktemp("sanitized")
    host = str(d / "libtp_host_double.so")
    orc = str(d / "liboracle_sanitized.so")
    subprocess.check_call(["g++", *SAN, "-std=c++20", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
                           os.path.join(ROOT, "tests", "host_double", "recorder.cpp"), "-o", host])
    subprocess.check_call(["gcc", *SAN, "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc, "-lm"])
    return host, orc


def test_oracle_and_abi_under_address_and_undefined_sanitizers(builds):
    host, orc = builds
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime("libasan.so"), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TP_HOST_DOUBLE_LIB=host,
               ORACLE_SANITIZED_LIB=orc, PYTHONPATH=ROOT, OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-rs", "-p", "no:cacheprovider", "-p", "tests.host_double.plugin",
           "-m", "not gpu", "tests/test_abi_cpu.py", "tests/test_oracle.py", "tests/test_oracle_attention.py",
           "tests/test_oracle_backward.py", "tests/host_double"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert "HOST DOUBLE VIOLATIONS: 0" in out
    # the recorded-launch tests ran (they skip only outside this run)
    assert "skipped" not in out and "test_launch_schedule" not in out.split("short test summary")[-1]
