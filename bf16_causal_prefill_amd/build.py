"""Builds libattn.so (the HIP kernels and the C-ABI entry points) for gfx950.

Run as `python -m bf16_causal_prefill_amd.build`.  Each .hip source is compiled
to an object in parallel, then linked into bf16_causal_prefill_amd/libattn.so.
`--phase-timers` builds libattn_phase_timers.so instead: the same sources with
ATTN_PHASE_TIMERS defined (shader-clock reads around the attention kernels' phases,
include/attn_phase_timers.h), a measurement build that the product never loads.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
TIMERS_LIB = os.path.join(PKG, "libattn_phase_timers.so")
SOURCES = ["api.hip", "attn_fwd_fp8.hip", "attn_fwd_bf16.hip", "merge.hip", "quantize.hip",
           "outliers.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


# The FP8 attention kernels produce no NaN from valid inputs (masking uses -inf, and
# every row sees key 0), so they are compiled without NaN semantics: otherwise the
# compiler puts a canonicalising max before each float max whose input it cannot prove
# quiet (IEEE signalling-NaN rules), 8 VALU instructions per tile in the FP8 matrix phase
# (+1-4% measured).  The BF16 kernels measured slower that way and keep the default.
PER_FILE_FLAGS = {"attn_fwd_fp8.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra: list[str], build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPFLAGS, *PER_FILE_FLAGS.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra: list[str] | None = None, verbose: bool = False, lib: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link `lib` (libattn.so); returns the library path."""
    os.makedirs(build_dir, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_phase_timers(verbose: bool = False) -> str:
    """The measurement build libattn_phase_timers.so (ATTN_PHASE_TIMERS defined)."""
    return build(["-DATTN_PHASE_TIMERS"], verbose, TIMERS_LIB,
                 os.path.join(BUILD, "phase_timers"))


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--phase-timers" in args:
        args.remove("--phase-timers")
        if args:
            raise SystemExit("--phase-timers takes no other arguments")
        build_phase_timers(verbose=True)
    else:
        build(args, verbose=True)
