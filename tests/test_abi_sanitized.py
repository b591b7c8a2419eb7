"""The C ABI's host code -- argument validation, 64-bit size arithmetic, workspace sizing,
the plan and its override, logging -- built with AddressSanitizer and
UndefinedBehaviorSanitizer (host pass only; the gfx950 code is unchanged) and exercised by
the CPU ABI tests in a child process that preloads the sanitizer runtime.  Any report
(out-of-bounds access, signed overflow, misaligned access, ...) aborts the child and fails
this test.  CPU only: nothing is launched."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Sanitizers on the host pass only, each flag preceded by -Xarch_host.
SANITIZE = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_abi_tests_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    sys.path.insert(0, ROOT)
    from online_softmax_attention_fa_amd import build as fa_build

    lib = str(tmp_path / "libfa_sanitized.so")
    fa_build.build(extra_flags=SANITIZE, link_flags=SANITIZE + ["-shared-libsan"], out=lib)
    env = dict(os.environ, FA_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "AddressSanitizer" not in out and "runtime error" not in out, out
