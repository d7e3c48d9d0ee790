"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every HIP source of the library with the sanitizers on the host pass only (the
gfx950 device code is compiled as usual and never runs here), links it with the driver
in tests/host_checks/abi_checks.cpp and runs that driver: a million seeded random
shapes - valid ones, ones at the 32-bit limits, invalid ones - through the sizing and
workspace-layout functions, each result checked against the bounds and region sizes the
header states, and every compute entry point with arguments it must reject before it
launches anything.  Needs no GPU.  A sanitizer report or a failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dropless_grouped_gemm_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_checks", "abi_checks.cpp")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"

# sanitizers on the host pass only: each -fsanitize= goes right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang++ not available")
    out = tmp_path_factory.mktemp("host_san")
    from dropless_grouped_gemm_amd.build import SOURCES
    common = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-Wno-pass-failed", "-Wno-inline-asm"] + HOST_SAN
    procs, objs = [], []
    for src in SOURCES:
        obj = str(out / src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append((src, subprocess.Popen(common + ["-c", os.path.join(CSRC, src), "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src, p in procs:
        text = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, f"{src}:\n{text[-4000:]}"
    drv = str(out / "abi_checks.o")
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "include"), "-c", DRIVER, "-o", drv], check=True)
    exe = str(out / "abi_checks")
    subprocess.run([CLANG, "-fsanitize=address,undefined", drv] + objs +
                   ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe], check=True)
    return exe


def test_abi_host_code_under_sanitizers(sanitized_driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, timeout=300, env=env)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-6000:]
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-6000:]
    assert "abi host checks: ok" in r.stdout
