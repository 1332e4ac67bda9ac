"""tests/test_abi.py once more, against libfdllm_asan.so: the same library with the host half of the C
ABI (api.hip: argument checks, status strings, handle checks) built with AddressSanitizer and
UndefinedBehaviorSanitizer.  It runs on the CPU, in a child process with clang's sanitizer runtime
preloaded ahead of anything already preloaded; any report ends the child with an error."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(lib, rt):
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(p for p in (rt, os.environ.get("LD_PRELOAD", "")) if p)
    env["FDLLM_LIB"] = lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def test_abi_under_host_sanitizers():
    from diffusion_long_context_amd.build import ASAN_LIB, asan_runtime
    if not os.path.exists(ASAN_LIB):
        pytest.fail("libfdllm_asan.so is not built: run `python -m diffusion_long_context_amd.build`")
    rt = asan_runtime()
    assert rt, "clang's AddressSanitizer runtime is missing from /opt/rocm/llvm"
    # the library really is instrumented: it calls into the sanitizer runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", ASAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = _env(ASAN_LIB, rt)
    # the child loads the sanitized build, not the plain one
    probe = ("from diffusion_long_context_amd.fdllm import load; load(); "
             "print(any('libfdllm_asan.so' in l for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("True"), r.stdout[-2000:] + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, r.stderr[-3000:]


def test_debug_variant_compiles(tmp_path):
    """The host half of the debug build (FDL_DEBUG: every call waits for its kernels and reports
    changes of the status word) compiles; the full variant is `build --debug`."""
    from diffusion_long_context_amd.build import CSRC, FLAGS, HIPCC, HOST_ABI_SOURCE
    r = subprocess.run([HIPCC, *FLAGS, "-DFDL_DEBUG", "-g", "-c", "-o", str(tmp_path / "api_debug.o"),
                        os.path.join(CSRC, HOST_ABI_SOURCE)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
