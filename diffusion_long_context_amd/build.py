"""Build libfdllm.so (all HIP sources for gfx950) in-tree.

Usage: python -m diffusion_long_context_amd.build [--phase-stamps] [--debug] [--out PATH]
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


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB) -> str:
    """Every source compiled to an object in parallel (relocatable device code is not needed: each
    kernel lives in one translation unit), then one link."""
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="fdllm_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[HIPCC, *FLAGS, *(extra or []), "-c", "-o", obj, src] for src, obj in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            results = list(pool.map(lambda c: _run(c, verbose), cmds))
        failed = [r for r in results if r.returncode != 0]
        if failed:
            for r in failed:
                sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed compiling libfdllm.so sources")
        tmp = out + ".tmp"
        r = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking libfdllm.so")
    os.replace(tmp, out)
    return out


def main(argv=None) -> str:
    import argparse
    ap = argparse.ArgumentParser(description="build libfdllm.so for gfx950")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="record the fused kernel's phase timestamps (diagnostic build)")
    ap.add_argument("--debug", action="store_true",
                    help="keep device-side assertions and host symbols (-O1 -g; FDL_DEBUG defined)")
    ap.add_argument("--out", default=None, help="library path (default: the in-tree libfdllm.so, or "
                                               "libfdllm_stamps.so / libfdllm_debug.so for the variants)")
    a = ap.parse_args(argv)
    extra, out = [], LIB
    if a.phase_stamps:
        extra.append("-DFDL_PHASE_STAMPS")
        out = os.path.join(HERE, "libfdllm_stamps.so")
    if a.debug:
        extra += ["-DFDL_DEBUG", "-g"]
        out = os.path.join(HERE, "libfdllm_debug.so")
    return build(verbose=True, extra=extra, out=a.out or out)


if __name__ == "__main__":
    print(main())
