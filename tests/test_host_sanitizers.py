"""Host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

libvsa's host code (problem validation, workspace planning, varlen and video
metadata, the 3-D tile partition, the error strings, the allocation-free
entry's size check) is compiled a second time with host-side ASan + UBSan
(``-Xarch_host`` keeps the device code uninstrumented), linked against the
shared sanitizer runtime, and every test of ``tests/test_abi_host.py`` is run
against that build in a child process that preloads the runtime.  Any
sanitizer report fails the test.  ``tests/cpp/layout_check.hip`` (the host
simulation of the attention kernel's LDS index maps) is built and run with
the same sanitizers.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# each -fsanitize= directly after -Xarch_host: host code only
SAN_COMPILE = ["-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-g"]
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}
REPORT_MARKS = ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer")


def _asan_runtime():
    hits = sorted(glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _clangxx():
    p = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
    return p if os.path.exists(p) else None


@pytest.fixture(scope="module")
def asan_lib():
    rt, cxx = _asan_runtime(), _clangxx()
    if rt is None or cxx is None:
        pytest.skip("ROCm clang sanitizer runtime not found")
    from video_sparse_attention_amd import build as B
    lib = os.path.join(ROOT, "_build", "asan", "libvsa_asan.so")
    link = [cxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan",
            f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    B.build(extra_flags=SAN_COMPILE, build_dir=os.path.join(ROOT, "_build", "asan"), lib_path=lib,
            link_cmd=link)
    return lib, rt


def _assert_clean(r):
    text = r.stdout + r.stderr
    for mark in REPORT_MARKS:
        assert mark not in text, text[-6000:]
    assert r.returncode == 0, text[-6000:]


def test_instrumented_library_links_the_sanitizer_runtime(asan_lib):
    lib, _ = asan_lib
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    assert "__asan_report_load8" in out or "__asan_loadN" in out or "__asan_report" in out
    assert "__ubsan_handle" in out


def test_host_abi_tests_under_sanitizers(asan_lib):
    lib, rt = asan_lib
    env = dict(os.environ, VSA_LIBRARY=lib, LD_PRELOAD=rt, **SAN_ENV)
    env.pop("PYTEST_ADDOPTS", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    _assert_clean(r)
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-3000:]


def test_layout_check_under_sanitizers(tmp_path):
    if _asan_runtime() is None:
        pytest.skip("ROCm clang sanitizer runtime not found")
    exe = tmp_path / "layout_check_asan"
    src = os.path.join(ROOT, "tests", "cpp", "layout_check.hip")
    inc = [f"-I{os.path.join(ROOT, 'video_sparse_attention_amd', 'csrc')}",
           f"-I{os.path.join(ROOT, 'include')}"]
    subprocess.run(["hipcc", "-O1", "-std=c++17", *SAN_COMPILE, *inc, src, "-o", str(exe)], check=True,
                   capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(os.environ, **SAN_ENV))
    _assert_clean(r)
    assert "layout checks passed" in r.stdout
