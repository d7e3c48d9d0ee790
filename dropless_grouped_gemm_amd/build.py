"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree, and its debug
variant libmoe_debug.so (MOE_DEBUG: the kernels' bounds checks also report what they
skip or clamp, read back with moe_debug_flags).

    python -m dropless_grouped_gemm_amd.build           # both
    python -m dropless_grouped_gemm_amd.build release   # libmoe.so only

Packed-fp32 instructions are disabled for all device code: the compiler would
otherwise form v_pk_* fp32 operations from ordinary float code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")
DEBUG_LIB = os.path.join(HERE, "libmoe_debug.so")
SOURCES = ["moe_api.hip", "moe_route.hip", "moe_offsets.hip", "moe_permute.hip", "moe_gemm.hip", "moe_gemm_wide.hip", "moe_fp8.hip", "moe_backward.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, arch: str = "gfx950", debug: bool = False) -> str:
    objdir = os.path.join(HERE, "_build_debug" if debug else "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc(), f"--offload-arch={arch}", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-Wno-pass-failed"]
    if debug:
        common.append("-DMOE_DEBUG")
    lib_path = DEBUG_LIB if debug else LIB
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = common + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature: harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={arch}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


def build_all(verbose: bool = False) -> None:
    """The release library and the debug variant."""
    build(verbose=verbose)
    build(verbose=verbose, debug=True)


if __name__ == "__main__":
    if "release" in sys.argv:
        print(build(verbose="-v" in sys.argv))
    else:
        build_all(verbose="-v" in sys.argv)
        print(LIB, DEBUG_LIB)
