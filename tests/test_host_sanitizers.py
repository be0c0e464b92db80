"""The host layer of the library under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

A host-only build of the C-ABI layer (``api.cpp`` with its validation,
planning and workspace sizing; the kernel launchers replaced by stand-ins
that refuse) is compiled with both sanitizers, every report fatal.  Then:

* the CPU library tests (``test_library_cpu.py``) run against it in a Python
  process with the sanitizer runtime preloaded;
* the row-chunk geometry checker (``tests/host/chunk_geometry.cpp``) is
  built and run with both sanitizers;
* the plain-C consumer is built with both sanitizers against it and runs its
  host checks.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CSRC = os.path.join(ROOT, "attention_score_selection_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
# Host code only is instrumented (each -fsanitize after -Xarch_host).
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def hipcc():
    path = os.path.join(ROCM, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def clang():
    path = os.path.join(ROCM, "llvm", "bin", "clang")
    return path if os.path.exists(path) else None


def asan_runtime():
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


pytestmark = pytest.mark.skipif(hipcc() is None or clang() is None or asan_runtime() is None,
                                reason="needs hipcc, ROCm's clang and its sanitizer runtime")


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    api_o, stub_o, lib = str(d / "api.o"), str(d / "stubs.o"), str(d / "libtsel_san.so")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, *SAN]
    run([hipcc(), *flags, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    run([hipcc(), *flags, "-c", os.path.join(HERE, "host", "launch_stubs.cpp"), "-o", stub_o])
    run([hipcc(), "-shared", "-fPIC", api_o, stub_o, "-o", lib])
    return lib


def test_library_cpu_tests_under_sanitizers(san_lib, tmp_path):
    env = dict(os.environ, TSEL_LIBRARY=san_lib, LD_PRELOAD=asan_runtime(), **SAN_ENV)
    env["ASAN_OPTIONS"] += f":log_path={tmp_path}/asan"
    env["UBSAN_OPTIONS"] += f":log_path={tmp_path}/ubsan"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_library_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-k", "not plain_c_and_cpp and not consumer"],
                       capture_output=True, text=True, env=env, timeout=900, cwd=ROOT)
    reports = [open(f).read() for f in glob.glob(str(tmp_path / "*san*"))]
    assert not reports, "\n".join(reports)[:6000]
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout


def test_chunk_geometry_under_sanitizers(tmp_path):
    exe = str(tmp_path / "chunk_geometry")
    run([hipcc(), "-O1", "-g", "-std=c++17", "-I", INCLUDE, "-I", CSRC, *SAN,
         os.path.join(HERE, "host", "chunk_geometry.cpp"), "-o", exe])
    r = run([exe], env=dict(os.environ, **SAN_ENV), timeout=120)
    assert r.stdout.startswith("ok"), r.stdout


def test_c_consumer_host_checks_under_sanitizers(san_lib, tmp_path):
    exe = str(tmp_path / "tsel_consumer")
    lib_dir = os.path.dirname(san_lib)
    os.symlink(san_lib, os.path.join(lib_dir, "libtsel.so"))
    run([clang(), "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
         os.path.join(HERE, "c_consumer", "tsel_consumer.c"), "-o", exe, "-L", lib_dir, "-ltsel",
         "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + lib_dir,
         "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    r = run([exe, "check"], env=dict(os.environ, **SAN_ENV), timeout=120)
    assert "check ok" in r.stdout
