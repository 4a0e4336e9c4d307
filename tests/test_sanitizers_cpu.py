"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host builds go to a temporary directory with -fsanitize=address,undefined
(every report fatal): the fp64 oracle (oracle/oracle.c), and the library's
host layer (abi.cpp and plan.cpp: argument checks, workspace and metadata
sizing, the hand-off to the launchers) linked with host stubs for the device
launchers (abi_host_stubs.cpp).  The oracle pins, the C-ABI checks and the
stubbed launch checks then run against them in a child pytest with the
sanitizer runtime preloaded; the child's exit status and output decide.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tenant_lora_serving_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    if not shutil.which("gcc") or not shutil.which("g++") or not _runtime():
        pytest.skip("gcc with the AddressSanitizer runtime is not available")
    d = tmp_path_factory.mktemp("san")
    oracle = str(d / "liboracle_san.so")
    host = str(d / "liblora_host_san.so")
    subprocess.run(["gcc", *SAN, "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle], check=True)
    subprocess.run(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
                    os.path.join(ROOT, "tests", "abi_host_stubs.cpp"), "-o", host], check=True)
    return oracle, host


def _child(files, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = _runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *files], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    for tag in ("ERROR: AddressSanitizer", "runtime error:"):
        assert tag not in out, out[-6000:]
    return out


def test_oracle_pins_under_sanitizers(builds):
    oracle, _ = builds
    out = _child(["tests/test_oracle_pins.py"], {"TL_TEST_ORACLE_LIB": oracle})
    assert " passed" in out


def test_c_abi_host_layer_under_sanitizers(builds):
    _, host = builds
    out = _child(["tests/test_abi_cpu.py", "tests/abi_stubbed_checks.py"],
                 {"TL_TEST_LORA_LIB": host, "TL_STUBBED_LORA_LIB": host})
    assert " passed" in out and "skipped" not in out
