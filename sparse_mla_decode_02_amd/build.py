"""Compile the HIP library (csrc/smla.hip -> libsmla.so) for gfx950 in-tree."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "smla.hip")
SRC_PAGED = os.path.join(HERE, "csrc", "smla_paged.hip")
SRC_FOURWAVE = os.path.join(HERE, "csrc", "smla_fourwave.hip")
LIB = os.path.join(HERE, "libsmla.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 arithmetic in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA results in VGPRs: the logit accumulators are read by vector
# instructions right after their MFMAs, which otherwise copy them out of AGPRs
# (64 instructions per tile).  Not for the paged instances (smla_paged.hip):
# there it makes registers spill into AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The first kernel arguments in SGPRs at wave start (the decode kernel's ten
# leading scalars, the combine kernel's six): no dependent kernel-argument load
# before a kernel's first memory requests.
PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=10"]
# The main unit (the pipelined decode kernel, the combine and per-head kernels,
# the host code) is scheduled for instruction-level parallelism: the pipelined
# kernel measured 0.4-0.5 us faster per step at 32 x 64 heads x top-512 (and
# ~1 us at top-2048); the four-wave kernel measured slower with it, so its
# contiguous instances (smla_fourwave.hip) and the paged ones (smla_paged.hip)
# keep the default scheduler.
SCHED_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
# The four-wave contiguous unit is scheduled to keep memory instructions in
# clauses: 0.4 us less decode at 96 x 16 heads x top-2048 in UE8M0 rows, the
# same at 64 x 64 heads; on the paged unit it measured 0.8 us slower at
# 64 x 64 heads, so that unit keeps the default.
SCHED_CLAUSE = ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsmla.so)")


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("building libsmla.so failed: " + " ".join(cmd[:1] + cmd[-3:]))
    if verbose:
        sys.stderr.write(res.stderr)


def build(verbose: bool = False, extra: list | None = None) -> str:
    """Always recompiles (three objects, then one shared library); writes to a
    temporary file then renames atomically."""
    tag = "%d" % os.getpid()
    tmp_dir = os.path.join(HERE, "_build_tmp" + tag)
    os.makedirs(tmp_dir, exist_ok=True)
    try:
        obj_main = os.path.join(tmp_dir, "smla.o")
        obj_fourwave = os.path.join(tmp_dir, "smla_fourwave.o")
        obj_paged = os.path.join(tmp_dir, "smla_paged.o")
        _run([hipcc(), *HIPCC_FLAGS, *VGPR_FORM, *PRELOAD, *SCHED_ILP, *(extra or []), "-c", SRC, "-o", obj_main],
             verbose)
        _run([hipcc(), *HIPCC_FLAGS, *VGPR_FORM, *PRELOAD, *SCHED_CLAUSE, *(extra or []), "-c", SRC_FOURWAVE, "-o",
              obj_fourwave], verbose)
        _run([hipcc(), *HIPCC_FLAGS, *PRELOAD, *(extra or []), "-c", SRC_PAGED, "-o", obj_paged], verbose)
        tmp = LIB + ".tmp" + tag
        _run([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", obj_main, obj_fourwave, obj_paged, "-o", tmp],
             verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmp_dir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
