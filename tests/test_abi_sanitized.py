"""The C-ABI layer under host AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library is rebuilt with both sanitizers on its host code
(argument checks, launch set-up; device code unchanged) and the whole C-ABI
suite (tests/test_abi.py: every entry point's argument checks, the exports,
the status strings) runs against it in a child process with the sanitizer
runtime preloaded. Any invalid access or undefined behaviour aborts that
process, which fails this test."""

import os
import subprocess
import sys

import pytest

from block_scaled_fp8_quant_amd import build as fbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_suite_under_host_sanitizers(tmp_path):
    try:
        runtime = fbuild.sanitizer_runtime()
        fbuild.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = fbuild.build_host_sanitized(str(tmp_path / "libfp8blk_hostsan.so"))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ, FP8BLK_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
