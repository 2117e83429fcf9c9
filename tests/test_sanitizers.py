"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

  * the oracle (oracle/oracle.c, gcc) runs the oracle's pins (tests/test_oracle.py
    without the planted-mistake copies, which are built and loaded on their own);
  * the library's host code (argument validation, launch plan, workspace sizing
    and the entry points' host paths in csrc/paged_attn.hip, compiled for the
    host only) runs the C-ABI boundary tests (tests/test_boundary.py).
Each runs in a child process with the matching sanitizer runtime preloaded; any
sanitizer report fails the test. No GPU code is built with a sanitizer.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer",
           "UndefinedBehaviorSanitizer")


def _run_pytest(test_file, env_extra, selector=None):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", test_file, "-q", "-x", "-p", "no:cacheprovider",
           "-m", "not gpu"]
    if selector:
        cmd += ["-k", selector]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    for r in REPORTS:
        assert r not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
                    "-o", str(lib), "-lm"], check=True)
    out = _run_pytest("tests/test_oracle.py",
                      {"PAGED_ATTN_ORACLE_LIB": str(lib), "LD_PRELOAD": asan},
                      selector="not planted_mistake")
    assert " passed" in out


def test_host_code_under_asan_and_ubsan(checked_build):
    lib, _ = checked_build
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout  # instrumented
    env = {"PAGED_ATTN_LIBRARY": lib, "LD_PRELOAD": rt[-1]}
    # the child loads this build, with the runtime in the process
    probe = subprocess.run(
        [sys.executable, "-c", "import paged_kv_gqa_decode_amd as pa; pa.library(); "
         "print(open('/proc/self/maps').read())"],
        cwd=ROOT, env={**os.environ, **env, "ASAN_OPTIONS": "detect_leaks=0"},
        capture_output=True, text=True)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert lib in probe.stdout and "libclang_rt.asan" in probe.stdout
    out = _run_pytest("tests/test_boundary.py", env)
    assert " passed" in out
