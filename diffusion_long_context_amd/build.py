"""Build libfdllm.so (all HIP sources for gfx950) in-tree.

Usage: python -m diffusion_long_context_amd.build [--phase-stamps] [--debug] [--no-sanitized] [--out PATH]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfdllm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 ops by itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> subprocess.CompletedProcess:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


# The host half of the C ABI (api.hip: argument checks, workspace carving, launch order) built a
# second time with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (the device
# code of a gfx950 library cannot take them); libfdllm_asan.so runs the ABI tests on the CPU with
# the sanitizer runtime preloaded.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
ASAN_LIB = os.path.join(HERE, "libfdllm_asan.so")
HOST_ABI_SOURCE = "api.hip"


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime that matches hipcc (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB,
          sanitized: str | None = None) -> str:
    """Every source compiled to an object in parallel (relocatable device code is not needed: each
    kernel lives in one translation unit), then one link.  sanitized: also link a library at that
    path whose api.hip object carries the host-side sanitizers (the other objects are shared)."""
    srcs = sources()
    jobs = max(1, min(len(srcs) + 1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="fdllm_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[HIPCC, *FLAGS, *(extra or []), "-c", "-o", obj, src] for src, obj in zip(srcs, objs)]
        api_src = os.path.join(CSRC, HOST_ABI_SOURCE)
        san_obj = os.path.join(tmpdir, "api_sanitized.o")
        if sanitized:
            cmds.append([HIPCC, *FLAGS, *(extra or []), *SANITIZE, "-g", "-c", "-o", san_obj, api_src])
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            results = list(pool.map(lambda c: _run(c, verbose), cmds))
        failed = [r for r in results if r.returncode != 0]
        if failed:
            for r in failed:
                sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed compiling libfdllm.so sources")
        links = [(out, objs)]
        if sanitized:
            links.append((sanitized, [san_obj if src == api_src else o for src, o in zip(srcs, objs)]))
        for path, lobjs in links:
            tmp = path + ".tmp"
            r = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *lobjs], verbose)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed linking {os.path.basename(path)}")
            os.replace(tmp, path)
    return out


def main(argv=None) -> str:
    import argparse
    ap = argparse.ArgumentParser(description="build libfdllm.so for gfx950")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="record the fused kernel's phase timestamps (diagnostic build)")
    ap.add_argument("--debug", action="store_true",
                    help="debug build (-g, FDL_DEBUG): every call waits for its kernels, so a failing "
                         "kernel is reported by the call that launched it, and changes of the status "
                         "word are printed on stderr with the launch that made them")
    ap.add_argument("--out", default=None, help="library path (default: the in-tree libfdllm.so, or "
                                               "libfdllm_stamps.so / libfdllm_debug.so for the variants)")
    ap.add_argument("--no-sanitized", action="store_true",
                    help="skip libfdllm_asan.so (api.hip with host-side ASan/UBSan)")
    a = ap.parse_args(argv)
    extra, out = [], LIB
    if a.phase_stamps:
        extra.append("-DFDL_PHASE_STAMPS")
        out = os.path.join(HERE, "libfdllm_stamps.so")
    if a.debug:
        extra += ["-DFDL_DEBUG", "-g"]
        out = os.path.join(HERE, "libfdllm_debug.so")
    variant = a.phase_stamps or a.debug or a.out
    return build(verbose=True, extra=extra, out=a.out or out,
                 sanitized=None if (variant or a.no_sanitized) else ASAN_LIB)


if __name__ == "__main__":
    print(main())
