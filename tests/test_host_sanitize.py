"""Host code under the address and undefined-behaviour sanitizers (CPU only).

* The C-ABI layer (csrc/bsl_api.cpp) is built with g++ together with a fake
  device (tests/host/fake_device.cpp: a gfx950 that reports itself, kernel
  launchers that only record what they were given) and driven by
  tests/host/abi_host_test.cpp, which creates plans and checks every argument
  error of every entry point, and that good calls reach the right launcher.
  Without a GPU this reaches far more of the layer than the real library can.
* The oracle (oracle/orc.c) is built with the same sanitizers and the oracle's
  pin tests run against that build (ORC_LIBRARY selects it).
* A planted heap overflow, built and loaded the same way, must be reported, so
  a silent sanitizer cannot pass these tests.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ORACLE_PINS = ["tests/test_oracle_forward.py", "tests/test_oracle_blocks.py",
               "tests/test_oracle_backward.py", "tests/test_oracle_window.py",
               "tests/test_oracle_kmer.py"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _runtime_env():
    """LD_PRELOAD of gcc's sanitizer runtimes, for shared objects loaded into
    an unsanitized interpreter."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                              text=True, check=True).stdout.strip()
        if not os.path.isabs(path) or not os.path.exists(path):
            pytest.skip(f"gcc has no {name}")
        libs.append(path)
    env = dict(os.environ, LD_PRELOAD=" ".join(libs), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return env


def test_abi_layer_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_host_test"
    cmd = ["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", *SAN, "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "block_sparse_local_amd", "csrc"),
           "-I", os.path.join(ROOT, "tests", "host"),
           os.path.join(ROOT, "block_sparse_local_amd", "csrc", "bsl_api.cpp"),
           os.path.join(ROOT, "tests", "host", "fake_device.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_host_test.cpp"), "-o", str(exe)]
    if not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("HIP headers not installed")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "liborc_san.so"
    subprocess.run(["gcc", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
                    "-D_POSIX_C_SOURCE=200809L", *SAN, os.path.join(ROOT, "oracle", "orc.c"),
                    "-o", str(lib), "-lm", "-lpthread"], check=True)
    env = dict(_runtime_env(), ORC_LIBRARY=str(lib))
    # the sanitized build is the one the oracle loads
    probe = ("import oracle, sys; lib = oracle.load(); "
             "sys.exit(0 if lib._name == sys.argv[1] else 5)")
    r = subprocess.run([sys.executable, "-c", probe, str(lib)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *ORACLE_PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "runtime error" not in r.stderr


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int poke(int n) { int *a = malloc(n * sizeof(int)); a[n] = 1;"
                   " int r = a[0]; free(a); return r; }\n")
    lib = tmp_path / "liboverflow.so"
    subprocess.run(["gcc", "-fPIC", "-shared", *SAN, str(src), "-o", str(lib)], check=True)
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).poke(4)"
    r = subprocess.run([sys.executable, "-c", code], env=_runtime_env(), capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
