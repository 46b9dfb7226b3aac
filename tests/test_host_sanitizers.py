"""The host C++ (KV-cache manager and host tier, dynamic batcher, request
planner and ABI validation) and the C oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc), under the host-logic tests: the allocator
and host-tier sequences checked byte for byte against the Python model and
the oracle, the batcher policy, plan validation and coverage, and the oracle
pins.  Kernel launchers are stand-ins in this build (tests/sanitize), so no
device call is made; any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "generative_recommender_sequence_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-g", "-O1"]


def _runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not installed")
    out = tmp_path_factory.mktemp("san")
    host = str(out / "libhstu_host_san.so")
    srcs = [os.path.join(CSRC, f) for f in ("kv_cache.cpp", "batcher.cpp", "hstu_abi.cpp", "timing.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"))
    cmd = (["g++", "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"] + SAN +
           ["-o", host] + srcs + [f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    orc = str(out / "liboracle_san.so")
    osrc = [os.path.join(ROOT, "oracle", f) for f in ("hstu_oracle.c", "kv_oracle.c")]
    r = subprocess.run(["gcc", "-std=gnu11", "-shared", "-fPIC", "-fopenmp", "-fno-fast-math"] + SAN +
                       ["-o", orc] + osrc + ["-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return host, orc


def test_host_code_and_oracle_under_asan_and_ubsan(sanitized_libs):
    host, orc = sanitized_libs
    env = dict(os.environ)
    env.update(HSTU_LIBRARY=host, ORACLE_LIBRARY=orc, OMP_NUM_THREADS="4",
               LD_PRELOAD=" ".join([_runtime("libasan.so"), _runtime("libubsan.so")]),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_kv_cache.py", "test_batcher.py", "test_abi.py", "test_oracle.py")]
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not candidate_row_list and not planted_mistake"] + tests
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
