"""Build step: compile the libmoe HIP/C++ sources for gfx950 into libmoe.so,
in-tree next to this file."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")

SOURCES = ["api.cpp", "slot_cache.cpp", "route.hip", "permute.hip", "q4_gemv.hip",
           "q4_grouped_mfma.hip", "shared_gemv.hip", "decode_fused.hip", "stage_copy.hip", "cache_device.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          # packed fp32 arithmetic is kept off for all device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Measurement variant (libmoe_measure.so): the library, with the fused decode
# kernel recording a per-stage timeline (MOE_DECODE_TIMELINE, see
# decode_fused.hip), the work-list GEMM a per-item timeline (MOE_GEMM_TIMELINE,
# see q4_grouped_mfma.hip), and known-bytes read kernels for scaling HBM
# counters (measure.hip).  Never loaded by the tests or the timing line.
MEASURE_LIB = os.path.join(HERE, "libmoe_measure.so")
MEASURE_DEFINES = {"decode_fused.hip": ["-DMOE_DECODE_TIMELINE"], "q4_grouped_mfma.hip": ["-DMOE_GEMM_TIMELINE"]}
MEASURE_SOURCES = ["measure.hip"]


def _compile(src: str, build_dir: str = BUILD, defines=None) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = (defines or {}).get(src, [])
    cmd = [HIPCC, *CFLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, measure: bool = False) -> str:
    """Compile every source for gfx950 and link libmoe.so (measure=True: the
    measurement variant libmoe_measure.so)."""
    build_dir = os.path.join(BUILD, "measure") if measure else BUILD
    out = MEASURE_LIB if measure else LIB
    defines = MEASURE_DEFINES if measure else None
    os.makedirs(build_dir, exist_ok=True)
    srcs = [s for s in SOURCES + (MEASURE_SOURCES if measure else []) if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True, measure="--measure" in sys.argv)
