"""GPU parity at the size limits of the C ABI: the largest head count, a long
list with many splits, and the largest sequence stride of each row format
(rows just below the 2^31-byte offset limit).  Marked ``gpu``.

For the largest strides the cache is several GB, so the oracle runs on a
compact cache holding the same rows in the same list order (the result
depends only on the selected rows and their order)."""

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_decode_02_amd as smla
from tests._gpu import compare, device_inputs, log, run_decode
from workloads import build_host_cache, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def reference(w):
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                    row_format=w.row_format)
    return out, lse


@pytest.mark.parametrize("nsplit", [1, 0, 5])
def test_256_heads(nsplit):
    log(f"case: 256 heads num_splits {nsplit}")
    w = make_workload(seed=501, batch=2, heads=256, topk=200, seqlens=[3000, 90], kv_seq_stride=3000,
                      structure="ragged", q_mult=2.0)
    ref_out, ref_lse = reference(w)
    out, lse = run_decode(w, num_splits=nsplit)
    compare(out, lse, ref_out, ref_lse, label=f"H256/ns{nsplit}")


@pytest.mark.parametrize("nsplit", [0, 256, 4096])
def test_long_list_many_splits(nsplit):
    # 8192 entries = 256 tiles; 4096 requested splits are clamped to 256
    log(f"case: top-8192 num_splits {nsplit}")
    w = make_workload(seed=502, batch=2, heads=16, topk=8192, seqlens=[20000, 9000], kv_seq_stride=20000,
                      structure="ragged", q_mult=4.0)
    assert smla.num_splits(w.batch, w.heads, w.topk, nsplit, w.kv_seq_stride) <= 256
    ref_out, ref_lse = reference(w)
    out, lse = run_decode(w, num_splits=nsplit)
    compare(out, lse, ref_out, ref_lse, label=f"k8192/ns{nsplit}")


@pytest.mark.parametrize("row_format", [0, 1])
def test_largest_sequence_stride(row_format):
    rb = 584 if row_format == 1 else 640
    stride = (2 ** 31 - 1) // rb                     # the largest the ABI accepts
    assert smla.num_splits(2, 16, 96, 0, stride, row_format) >= 1
    assert smla.num_splits(2, 16, 96, 0, stride + 1, row_format) == -1
    log(f"case: largest stride {stride} rows, row format {row_format}")
    # compact twin: the same rows at positions 0..95 of a 96-row stride
    small = make_workload(seed=503, batch=2, heads=16, topk=96, seqlen=96, q_mult=2.0, row_format=row_format)
    small.idx[:] = np.arange(96)[None, :]            # list j selects row j
    small.idx[1, 7::9] = -1                          # a few masked entries
    ref_out, ref_lse = reference(small)
    # the large cache: row j of the list placed at position stride - 96 + perm(j)
    rng = np.random.default_rng(4)
    pos = (stride - 96 + rng.permutation(96)).astype(np.int64)
    q = torch.from_numpy(small.q_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    cache = torch.full((2 * stride, rb), 0xFF, dtype=torch.uint8, device=DEV)
    for b in range(2):
        cache[torch.from_numpy(b * stride + pos).to(DEV)] = torch.from_numpy(
            np.ascontiguousarray(small.rows[b])).to(DEV)
    idx = np.where(small.idx >= 0, pos[np.maximum(small.idx, 0)], -1).astype(np.int32)
    idx_d = torch.from_numpy(idx).to(DEV)
    seqlens = torch.full((2,), stride, dtype=torch.int32, device=DEV)
    for ns in (1, 2):
        out = torch.full((2, 16, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((2, 16), float("nan"), device=DEV)
        smla.sparse_mla_decode(q, cache, idx_d, seqlens, small.scale, out, lse, num_splits=ns, kv_seq_stride=stride,
                               row_format=row_format)
        torch.cuda.synchronize()
        compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out,
                ref_lse, label=f"stride {stride} fmt{row_format} ns{ns}")
    del cache
    torch.cuda.empty_cache()


def test_entries_past_the_stride_are_skipped():
    # seqlens above the stride: the decode and the per-head kernels skip the
    # entries at or past the stride instead of reading the next sequence
    w = make_workload(seed=504, batch=3, heads=32, topk=96, seqlen=400, kv_seq_stride=400)
    cache_h = build_host_cache(w)
    idx_bad = w.idx.copy()
    idx_bad[:, ::4] = 400 + np.arange(idx_bad[:, ::4].shape[1])[None, :]
    idx_ref = idx_bad.copy()
    idx_ref[:, ::4] = -1
    ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache_h, 400, idx_ref, w.seqlens, w.heads, w.scale)
    q, cache, _, _ = device_inputs(w)
    idx = torch.from_numpy(idx_bad).to(DEV)
    big = torch.full((3,), 10 ** 6, dtype=torch.int32, device=DEV)
    for kernel, ns in (("decode", 1), ("decode", 3), ("per-head", 0)):
        log(f"case: entries past the stride, {kernel} ns {ns}")
        out = torch.full((3, 32, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((3, 32), float("nan"), device=DEV)
        if kernel == "decode":
            smla.sparse_mla_decode(q, cache, idx, big, w.scale, out, lse, num_splits=ns, kv_seq_stride=400)
        else:
            smla.sparse_mla_decode_per_head(q, cache, idx, big, w.scale, out, lse, kv_seq_stride=400)
        torch.cuda.synchronize()
        compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_out,
                ref_lse, label=f"past stride {kernel} ns{ns}")
