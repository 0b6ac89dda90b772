"""GPU test of sparse_mla_decode_noalloc through the C ABI: its result equals
sparse_mla_decode's (same kernels, so bitwise) on two calls in a row, the
second with a smaller input, and both match the fp64 oracle to the parity
bar."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_decode_02_amd as smla
from tests._gpu import compare, device_inputs, log
from workloads import build_host_cache, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(w, inputs, num_splits):
    q, cache, idx, seqlens = inputs
    B, H = w.batch, w.heads
    out = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    shape = smla.make_shape(B, H, w.topk, num_splits, w.kv_seq_stride, w.row_format)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = smla.lib().sparse_mla_decode_noalloc(P(q), P(cache), P(idx), P(seqlens), ctypes.c_float(w.scale),
                                              P(out), P(lse), ctypes.byref(shape),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, smla.status_str(st)
    torch.cuda.synchronize()
    return out, lse


def _with_workspace(w, inputs, num_splits):
    q, cache, idx, seqlens = inputs
    B, H = w.batch, w.heads
    out = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    smla.sparse_mla_decode(q, cache, idx, seqlens, w.scale, out, lse, num_splits=num_splits,
                           kv_seq_stride=w.kv_seq_stride, row_format=w.row_format)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("row_format", [0, 1])
def test_noalloc_matches_workspace_entry_point(row_format):
    # first call: 16 sequences x 64 heads, 4 splits (8.4 MB of partials, most of
    # the scratch); second call: a smaller ragged input with 2 splits, which
    # reuses the scratch the first call left filled
    cases = [
        (dict(seed=41, batch=16, heads=64, topk=512, seqlen=8192, row_format=row_format), 4),
        (dict(seed=42, batch=3, heads=32, topk=100, seqlens=[300, 50, 7], kv_seq_stride=300,
              structure="ragged", q_mult=2.0, row_format=row_format), 2),
    ]
    for kw, ns in cases:
        log(f"case: noalloc {kw} num_splits {ns}")
        w = make_workload(**kw)
        got = smla.num_splits(w.batch, w.heads, w.topk, ns, w.kv_seq_stride, row_format)
        assert got == ns, (got, ns)
        inputs = device_inputs(w)
        out_n, lse_n = _noalloc(w, inputs, ns)
        out_w, lse_w = _with_workspace(w, inputs, ns)
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
        assert torch.equal(lse_n.view(torch.int32), lse_w.view(torch.int32))
        cache = build_host_cache(w)
        ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                                                w.scale, row_format=row_format)
        compare(out_n.float().cpu().numpy().astype(np.float64), lse_n.cpu().numpy().astype(np.float64),
                ref_out, ref_lse, label=f"noalloc/fmt{row_format}/B{w.batch}")
