"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_gqa_decode_pkv_amd.build [--asm]

Host-only C++ (planner, policy) and the HIP kernels link into one shared
library next to this file.  ``--asm`` also writes the gfx950 assembly of the
kernels under ``_build/`` for inspection.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for every device compile.  The
# atomic optimizer is off too: the decode kernel issues one counter atomic
# per task from one lane and consumes it a whole task later, and the
# optimizer's broadcast of the result would force an immediate wait on every
# load in flight.  The first two kernel arguments are preloaded into SGPRs
# (the decode kernel's task list and its capacity), so the first record load
# leaves at entry without a round trip to the argument segment.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                "-mllvm", "-amdgpu-kernarg-preload-count=2"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)


# Host-side sanitizers for the CPU checks of the planner, the policy, the
# runner and the entry points' argument handling (sanitize=True).  Every
# -fsanitize= goes to the host compilation only (-Xarch_host): the device code
# of the kernels is built as usual.  The result is a separate library under
# _build/sanitize/, loaded through PKV_LIB_PATH with the clang ASan runtime
# preloaded (see paged_gqa_decode_pkv_amd/sanitize.py); it is never run on a GPU.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


# The per-workgroup timeline (-DPKV_TIMELINE): the same kernels with
# realtime-counter marks kept in registers and stored once per workgroup at
# its exit, and pkv_timeline_read to fetch them.  A separate library beside
# the product one (libpkv_timeline.so; objects under _build/timeline/),
# loaded by timeline.py in place of the product library, which never
# contains the marks.
TIMELINE_FLAGS = ["-DPKV_TIMELINE"]
TIMELINE_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv_timeline.so")


def build(verbose: bool = False, asm: bool = False, sanitize: bool = False,
          timeline: bool = False) -> str:
    if sanitize and timeline:
        raise ValueError("the sanitizer and timeline builds are separate libraries")
    hipcc = _hipcc()
    out_dir = BUILD_DIR
    if sanitize:
        out_dir = os.path.join(BUILD_DIR, "sanitize")
    elif timeline:
        out_dir = os.path.join(BUILD_DIR, "timeline")
    os.makedirs(out_dir, exist_ok=True)
    common = ["-O1" if sanitize else "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-Wall"]
    if sanitize:
        common += SANITIZE_FLAGS
    objs = []
    plan_o = os.path.join(out_dir, "plan.o")
    # The policy's cost model must round every product and sum on its own
    # (its decisions are compared bit for bit with the reference): no FMA
    # contraction in the host planner.
    _run([hipcc, "-x", "c++", *common, "-ffp-contract=off", "-c",
          os.path.join(CSRC, "plan.cpp"), "-o", plan_o], verbose)
    objs.append(plan_o)
    run_o = os.path.join(out_dir, "runner.o")
    rocm_inc = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "include")
    _run([hipcc, "-x", "c++", *common, "-D__HIP_PLATFORM_AMD__", "-I", rocm_inc, "-c",
          os.path.join(CSRC, "runner.cpp"), "-o", run_o], verbose)
    objs.append(run_o)
    dec_o = os.path.join(out_dir, "decode.o")
    _run([hipcc, "-x", "hip", f"--offload-arch={ARCH}", *common, *DEVICE_FLAGS,
          *(TIMELINE_FLAGS if timeline else []), "-c",
          os.path.join(CSRC, "decode.hip"), "-o", dec_o], verbose)
    objs.append(dec_o)
    if asm and not (sanitize or timeline):
        _run([hipcc, "-x", "hip", f"--offload-arch={ARCH}", *common, *DEVICE_FLAGS,
              "--cuda-device-only", "-S", os.path.join(CSRC, "decode.hip"),
              "-o", os.path.join(BUILD_DIR, "decode-gfx950.s")], verbose)
    if sanitize:
        lib = os.path.join(out_dir, "libpkv.so")
    elif timeline:
        lib = TIMELINE_LIB
    else:
        lib = LIB
    tmp = lib + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", *(SANITIZE_FLAGS if sanitize else []),
          *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="host-side ASan/UBSan build under _build/sanitize/ (CPU checks only)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup timeline build, libpkv_timeline.so (timeline.py)")
    args = ap.parse_args()
    print(build(verbose=args.verbose, asm=args.asm, sanitize=args.sanitize,
                timeline=args.timeline))
