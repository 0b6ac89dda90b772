"""GPU parity of the per-head SIMT ablation kernel (one wave per (sequence,
head), rows re-read per head) against the fp64 CPU oracle.  Marked ``gpu``."""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_decode_02_amd as smla
from tests._gpu import compare, device_inputs, log
from workloads import build_host_cache, config_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_per_head(w, inputs=None):
    q, cache, idx, sl = inputs if inputs is not None else device_inputs(w)
    out = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((w.batch, w.heads), float("nan"), dtype=torch.float32, device=q.device)
    smla.sparse_mla_decode_per_head(q, cache, idx, sl, w.scale, out, lse, kv_seq_stride=w.kv_seq_stride,
                                    row_format=w.row_format)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def reference(w):
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                    row_format=w.row_format)
    return out, lse


@pytest.mark.parametrize("cfg,row_format", [(1, 0), (2, 0), (3, 0), (3, 1), (4, 0), (5, 0)])
def test_per_head_config_parity(cfg, row_format):
    log(f"case: per-head config {cfg} row format {row_format}")
    w = config_workload(cfg, row_format=row_format)
    ref_out, ref_lse = reference(w)
    out, lse = run_per_head(w)
    compare(out, lse, ref_out, ref_lse, label=f"per-head cfg{cfg}/fmt{row_format}")


@pytest.mark.parametrize("heads,topk", [(16, 45), (48, 1), (128, 100)])
def test_per_head_ragged_and_masked(heads, topk):
    log(f"case: per-head heads {heads} topk {topk}")
    w = make_workload(seed=400 + heads + topk, batch=3, heads=heads, topk=topk, seqlens=[300, 50, 7],
                      kv_seq_stride=300, structure="ragged", q_mult=4.0)
    w.idx[0, ::3] = -1
    ref_out, ref_lse = reference(w)
    out, lse = run_per_head(w)
    compare(out, lse, ref_out, ref_lse, label=f"per-head H{heads}/k{topk}")


def test_per_head_empty_list():
    w = make_workload(seed=410, batch=2, heads=16, topk=8, seqlens=[0, 10], kv_seq_stride=10)
    w.idx[1] = -1
    out, lse = run_per_head(w)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
