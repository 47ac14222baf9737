"""The library's host code (api.cpp, slot_cache.cpp) under AddressSanitizer,
UndefinedBehaviorSanitizer and LeakSanitizer, on the CPU.

The two host sources are compiled host-only (no device code is generated) and
linked with stand-ins for the HIP runtime and for the kernel launchers
(tests/host_sanitize/stub_*.cpp); tests/host_sanitize/driver.cpp then drives
the argument checks of every entry point, the expert cache in every staging
mode and eviction policy, and a HIP failure injected at each runtime call of
every staged step and of the cache's set-up calls.  Any sanitizer report, leak
or failed check makes the program exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
CSRC = os.path.join(REPO, "int4_routed_expert_route_amd", "csrc")
HS = os.path.join(HERE, "host_sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"

# Sanitizers on the host pass only (the sources are compiled host-only anyway).
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not present")
def test_host_code_under_sanitizers(tmp_path):
    objs = []
    for src in ("api.cpp", "slot_cache.cpp"):
        o = str(tmp_path / (src + ".o"))
        _run([HIPCC, "-x", "hip", "--cuda-host-only", *COMMON, *HOST_SAN, "-w", "-c",
              os.path.join(CSRC, src), "-o", o], str(tmp_path))
        objs.append(o)
    for src in ("stub_runtime.cpp", "stub_kernels.cpp", "driver.cpp"):
        o = str(tmp_path / (src + ".o"))
        _run([CLANG, *COMMON, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", os.path.join(HS, src), "-o", o],
             str(tmp_path))
        objs.append(o)
    exe = str(tmp_path / "driver")
    _run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe], str(tmp_path))
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], cwd=str(tmp_path), capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-8000:]
    assert "host checks passed" in r.stdout
    shutil.rmtree(str(tmp_path), ignore_errors=True)
