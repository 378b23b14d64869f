"""Compile the gfx950 HIP sources under csrc/ into libgbw.so (in-tree).

Every .hip file is compiled to an object in parallel with hipcc, then linked
into one shared library next to this file.  Flags:
  --offload-arch=gfx950               MI355X only, no other targets
  -ffp-contract=off                   no fused multiply-add contraction: the
                                      quantizers' fp32 steps round one by one
  -fhip-fp32-correctly-rounded-divide-sqrt, -fno-gpu-flush-denormals-to-zero
                                      IEEE division and subnormals, as the
                                      quantizer definitions assume
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      no packed fp32 VALU instructions
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgbw.so")
# measurement aid: the same sources with the MoE tile timeline compiled in
TRACE_LIB = os.path.join(HERE, "libgbw_tiletrace.so")
# measurement aid for the benchmark (a plain streaming read), its own library
FLOOR_SRCS = [os.path.join(HERE, "floor", f) for f in ("stream_read.hip", "mfma_rate.hip")]
FLOOR_LIB = os.path.join(HERE, "libgbw_floor.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = FLOOR_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", *FLOOR_SRCS, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {FLOOR_SRCS}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, FLOOR_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources, and {FLOOR_LIB}")
    return LIB


def build_tile_trace(verbose=False):
    """The library with the per-tile wall-clock stamps of the FP4 MoE kernel
    compiled in (-DGBW_TILE_TRACE), as libgbw_tiletrace.so; loaded only when
    GBW_LIBRARY names it (bench.py --part tiletrace)."""
    bdir = BUILD + "_trace"
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, bdir, ("-DGBW_TILE_TRACE",)), srcs))
    tmp = TRACE_LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, TRACE_LIB)
    if verbose:
        print(f"built {TRACE_LIB}")
    return TRACE_LIB


if __name__ == "__main__":
    if "--tile-trace" in sys.argv[1:]:
        build_tile_trace(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
