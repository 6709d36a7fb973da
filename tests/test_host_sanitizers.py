"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code only (each
-fsanitize flag behind -Xarch_host; the gfx950 device code is built as usual),
and the C-ABI test module (tests/test_abi.py: symbol export, host-only
functions, every validation path, the no-device path) runs against it in a
child process with the sanitizer runtime preloaded and every report fatal.
No GPU is used.
"""

import glob
import os
import subprocess
import sys

import pytest

from fp8_block_scaled_nt_amd import build as B

ROOT = B.ROOT


def _asan_runtime():
    pats = ["/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm*/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"]
    for p in pats:
        hits = sorted(glob.glob(p))
        if hits:
            return hits[-1]
    return None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    out = str(tmp_path_factory.mktemp("asan") / "libdg_asan.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), os.path.join(B.CSRC, "dg_api.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out, runtime


def test_sanitized_build_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms or "__asan_loadN" in syms
    assert "__ubsan_handle_" in syms


def test_abi_suite_clean_under_sanitizers(sanitized_lib):
    lib, runtime = sanitized_lib
    env = dict(os.environ)
    env.update({"DG_LIBRARY": lib, "LD_PRELOAD": runtime,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert " passed" in text
