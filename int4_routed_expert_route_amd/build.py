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


# Measurement variant: the fused decode kernel records a per-stage timeline
# (MOE_DECODE_TIMELINE, see decode_fused.hip); everything else is the library.
TIMELINE_LIB = os.path.join(HERE, "libmoe_timeline.so")
TIMELINE_DEFINES = {"decode_fused.hip": ["-DMOE_DECODE_TIMELINE"]}


def _compile(src: str, build_dir: str = BUILD, defines=None) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = (defines or {}).get(src, [])
    cmd = [HIPCC, *CFLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile every source for gfx950 and link libmoe.so (timeline=True: the
    measurement variant libmoe_timeline.so)."""
    build_dir = os.path.join(BUILD, "timeline") if timeline else BUILD
    out = TIMELINE_LIB if timeline else LIB
    defines = TIMELINE_DEFINES if timeline else None
    os.makedirs(build_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
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
    build(verbose=True, timeline="--timeline" in sys.argv)
