"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host code (argument checks, planning, the launch table, the
workspace and counter limits, the recurrent update's checks and byte
accounting) and the oracle's C code are rebuilt with both sanitizers, and the
CPU tests that exercise them run again against those builds, in child
processes that preload the matching sanitizer runtime (clang's for the
library, gcc's for the oracle). The device code of the library build is
compiled as usual: every sanitizer flag of its compile line is a host-only
flag. A sanitizer report ends the child with a non-zero status.
"""
import glob
import os
import subprocess
import sys

import pytest

from skinny_bit_block_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = lib_build.HIPCC

# the CPU tests that call into the library's host code / the oracle's C code
LIBRARY_TESTS = ["tests/test_abi.py", "tests/test_plan_table.py", "tests/test_gdn_host.py",
                 "tests/test_int4_host.py", "tests/test_nvfp4_host.py", "tests/test_plan_properties.py",
                 "tests/test_run_properties.py"]
ORACLE_TESTS = ["tests/test_oracle.py", "tests/test_oracle_ids.py"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def gcc_asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def run_tests(files, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", *files],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    for r in REPORTS:
        assert r not in out, out[-4000:]
    return out


@pytest.fixture(scope="module")
def library_build(tmp_path_factory):
    rt = clang_asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("no hipcc / clang AddressSanitizer runtime")
    out = str(tmp_path_factory.mktemp("asan") / "libqmm_asan.so")
    host = []
    for f in ("-O1", "-g", "-fno-omit-frame-pointer", "-shared-libsan",
              "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        host += ["-Xarch_host", f]
    cmd = ([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
            "-Xarch_device", "-O1",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"] + host +
           [os.path.join(lib_build.CSRC, s) for s in lib_build.SOURCES] + ["-o", out])
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-4000:]
    return out, rt


@pytest.fixture(scope="module")
def oracle_build(tmp_path_factory):
    rt = gcc_asan_runtime()
    if rt is None:
        pytest.skip("no gcc AddressSanitizer runtime")
    out = str(tmp_path_factory.mktemp("asan") / "liboracle_asan.so")
    src = os.path.join(ROOT, "oracle", "qk_oracle.c")
    res = subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-shared",
                          "-fPIC", "-std=c99", "-fsanitize=address,undefined",
                          "-fno-sanitize-recover=all", "-o", out, src, "-lm"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    return out, rt


def test_library_host_code_under_sanitizers(library_build):
    lib, rt = library_build
    out = run_tests(LIBRARY_TESTS, {"QMM_LIBRARY": lib, "LD_PRELOAD": rt})
    assert " passed" in out


def test_oracle_under_sanitizers(oracle_build):
    lib, rt = oracle_build
    out = run_tests(ORACLE_TESTS, {"ORACLE_LIBRARY": lib, "LD_PRELOAD": rt})
    assert " passed" in out


def test_sanitizer_builds_are_the_ones_loaded(library_build, oracle_build):
    # the overrides really select the sanitizer builds (a child that loads the
    # default libraries would pass the runs above without checking anything)
    lib, rt = library_build
    code = ("import skinny_bit_block_amd as s, ctypes; s.load(); "
            "print([l for l in open('/proc/self/maps').read().split() if l.endswith('.so')])")
    env = dict(os.environ, QMM_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    assert lib in res.stdout and "skinny_bit_block_amd/libqmm.so" not in res.stdout
    olib, ort = oracle_build
    code = ("import oracle; oracle.f16_to_f64(0x3C00); "
            "print([l for l in open('/proc/self/maps').read().split() if l.endswith('.so')])")
    env = dict(os.environ, ORACLE_LIBRARY=olib, LD_PRELOAD=ort, ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    assert olib in res.stdout and "oracle/liboracle.so" not in res.stdout
