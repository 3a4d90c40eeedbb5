"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host-side code,
exercised by the existing tests, on the CPU:

  * the C-ABI validation layer (global_attention_mimo_amd/csrc/api.cpp: every
    argument check, size computation and error mapping, and check mode's
    rules and gate) built with g++ and the sanitizers, linked with host-only
    launcher stand-ins (tests/sanitize/launch_stub.cpp), and loaded by
    tests/test_abi.py through MIMO_ATTN_LIBRARY and by
    tests/test_check_mode.py through MIMO_ATTN_HOST_STUB;
  * the fp64 oracle (oracle/mimo_oracle.c) built with gcc and the sanitizers
    and run against every pin of tests/oracle_pins.py.

Each runs in a child Python with the sanitizer runtime preloaded; any report
aborts the child, so the test fails on any sanitizer finding.  Leak checking is
off (the interpreter itself keeps allocations until exit).
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _env(**extra):
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(extra)
    return env


def test_validation_layer_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libmimo_attn_sanitized.so")
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "global_attention_mimo_amd", "csrc", "api.cpp"),
           os.path.join(HERE, "sanitize", "launch_stub.cpp"), "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
           "-lamdhip64", "-o", lib]
    subprocess.run(cmd, check=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan" in nm and "__ubsan" in nm, "the validation layer was not instrumented"
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"),
                          os.path.join(HERE, "test_check_mode.py"), "-q", "-x", "-p", "no:cacheprovider"], cwd=ROOT,
                         capture_output=True, text=True, timeout=600,
                         env=_env(MIMO_ATTN_LIBRARY=lib, MIMO_ATTN_HOST_STUB=lib))
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libmimo_oracle_sanitized.so")
    oracle.build(oracle.SOURCE, lib, extra_flags=tuple(SAN))
    res = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib], cwd=ROOT, capture_output=True,
                         text=True, timeout=900, env=_env(OMP_NUM_THREADS="4"))
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    failed = [l for l in res.stdout.splitlines() if l.startswith("FAILED:")]
    assert failed == ["FAILED:"], f"pins failing under the sanitizers: {failed}"
