"""GPU test of the SMLA_DEBUG_VALIDATE input scan: a child process with the
scan switched on runs decode calls (contiguous, paged, per-head) on inputs
with planted conditions; each call must report exactly the conditions its
inputs hold, and its results must still match the fp64 oracle.  Marked
``gpu``."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from tests._debug_cases import cases, expected_flags
from tests._gpu import compare, log
from workloads import build_host_cache, build_host_pool

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def reference(w, lay):
    if lay is None:
        out, lse, _ = oracle.decode_raw(w.q_bits, build_host_cache(w), w.kv_seq_stride, w.idx, w.seqlens,
                                        w.heads, w.scale)
    else:
        out, lse, _ = oracle.decode_paged_raw(w.q_bits, build_host_pool(w, lay), lay.num_pages, lay.page_size,
                                              lay.block_table, w.idx, w.seqlens, w.heads, w.scale)
    return out, lse


def test_debug_validate_reports_planted_conditions(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    path = tmp_path / "debug.npz"
    env = dict(os.environ, SMLA_DEBUG_VALIDATE="1", PYTHONPATH=ROOT)
    log("starting the debug-validate child process")
    r = subprocess.run([sys.executable, "-u", "-m", "tests._debug_child", str(path)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    log(r.stdout[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    got = np.load(path)
    for name, kind, w, lay in cases():
        flags = int(got[f"{name}.flags"])
        assert flags == expected_flags(w, lay), (name, flags)
        ref_out, ref_lse = reference(w, lay)
        compare(got[f"{name}.out"], got[f"{name}.lse"], ref_out, ref_lse, label=f"debug-validate {name}")
