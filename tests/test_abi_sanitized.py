"""The CPU ABI checks (tests/test_abi_host.py) once more, against a build of
the library whose host code carries AddressSanitizer and UndefinedBehavior-
Sanitizer instrumentation (the device code is built as usual and never runs
here).  Any sanitizer report fails the test.

The instrumented library is built in a temporary folder; the checks run in a
child process with the compiler's ASan runtime preloaded (Python itself is not
instrumented), and the test fixture loads that library in place of the
regular one through MOE_ABI_TEST_LIB."""
import glob
import importlib.util
import os
import subprocess
import sys
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_mod():
    spec = importlib.util.spec_from_file_location(
        "moe_mi355x_build", os.path.join(ROOT, "mixture_experts_ffn_07_amd", "build.py"))
    B = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(B)
    return B


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    B = _build_mod()
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if _asan_runtime() is None:
        pytest.skip("no clang ASan runtime")
    out = tmp_path_factory.mktemp("asan")
    # sanitizers for the host pass only (each -fsanitize behind -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include")] + san

    def compile_one(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([hipcc] + flags + ["-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = str(out / "libmoe_host_sanitized.so")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan"] +
                       san + objs + ["-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib


def test_abi_checks_under_asan_and_ubsan(sanitized_lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), MOE_ABI_TEST_LIB=sanitized_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in r.stdout
