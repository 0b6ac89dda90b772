"""GPU parity for the paged cache (rows in a shuffled pool of pages, found
through a per-sequence block table): libsmla.so through its C ABI against the
fp64 CPU oracle on the same seeded inputs.  Marked ``gpu``.

For the large workloads the reference is the oracle on the contiguous cache
holding the same rows, which the CPU tests pin bit for bit to the oracle's
paged form (tests/test_oracle.py::test_paged_equals_contiguous_bitwise)."""

import functools

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_decode_02_amd as smla
from tests._gpu import compare, log
from workloads import (build_host_cache, build_host_pool, config_workload, make_paged_layout,
                       make_workload, physical_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def device_paged_inputs(w, lay):
    """q, pool uint8 [num_pages * page_size, row bytes] (0xFF except kept rows),
    block table, idx, seqlens on the GPU."""
    q = torch.from_numpy(w.q_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    pool = torch.full((lay.num_pages * lay.page_size, w.row_bytes), 0xFF, dtype=torch.uint8, device=DEV)
    phys = physical_rows(w, lay)
    b_i, j_i = np.nonzero(phys >= 0)    # rows that a page of the pool holds
    assert phys.max(initial=-1) < lay.num_pages * lay.page_size
    if len(b_i):
        pool[torch.from_numpy(phys[b_i, j_i]).to(DEV)] = torch.from_numpy(
            np.ascontiguousarray(w.rows[b_i, j_i])).to(DEV)
    bt = torch.from_numpy(lay.block_table).to(DEV)
    return q, pool, bt, torch.from_numpy(w.idx).to(DEV), torch.from_numpy(w.seqlens).to(DEV)


def run_paged(w, lay, inputs=None, num_splits=0, idx=None):
    q, pool, bt, idx0, sl = inputs if inputs is not None else device_paged_inputs(w, lay)
    idx = idx0 if idx is None else idx
    out = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.batch, w.heads), float("nan"), dtype=torch.float32, device=DEV)
    smla.sparse_mla_decode_paged(q, pool, bt, idx, sl, w.scale, out, lse, page_size=lay.page_size,
                                 num_pages=lay.num_pages, num_splits=num_splits, row_format=w.row_format)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@functools.lru_cache(maxsize=1)
def contiguous_reference(cfg, row_format):
    log(f"building workload config {cfg} (row format {row_format}) and its oracle")
    w = config_workload(cfg, row_format=row_format)
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                    row_format=row_format)
    return w, out, lse


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    contiguous_reference.cache_clear()


# grouped by (config, row format) so that each reference is built once
CASES = [(1, 0, 16, 1), (1, 0, 1, 2), (1, 1, 256, 0),
         (2, 0, 64, 0), (2, 0, 1, 4),
         (3, 0, 64, 0), (3, 0, 16, 1), (3, 0, 1, 0),
         (3, 1, 64, 0),
         (4, 0, 64, 0),
         (5, 0, 64, 0)]


@pytest.mark.parametrize("cfg,row_format,page_size,nsplit", CASES)
def test_paged_config_parity(cfg, row_format, page_size, nsplit):
    log(f"case: paged config {cfg} row format {row_format} page {page_size} num_splits {nsplit}")
    w, ref_out, ref_lse = contiguous_reference(cfg, row_format)
    lay = make_paged_layout(w, page_size, seed=cfg + page_size, spare_pages=7)
    out, lse = run_paged(w, lay, num_splits=nsplit)
    compare(out, lse, ref_out, ref_lse, label=f"paged cfg{cfg}/fmt{row_format}/page{page_size}/ns{nsplit}")


@pytest.mark.parametrize("row_format", [0, 1])
def test_paged_against_paged_oracle_with_missing_pages(row_format):
    # block-table slots that are -1, negative, past the pool, and positions past
    # the table row: the kernel must skip exactly the entries the oracle skips
    w = make_workload(seed=301, batch=4, heads=64, topk=300, seqlens=[2000, 700, 40, 2000],
                      kv_seq_stride=2000, structure="ragged", q_mult=2.0, row_format=row_format)
    lay = make_paged_layout(w, 32, seed=5, spare_pages=9, all_pages=True)
    bt = lay.block_table.copy()
    bt[0, 3], bt[0, 11], bt[1, 2], bt[3, 0] = -1, -77, lay.num_pages, lay.num_pages + 1000
    bt = np.ascontiguousarray(bt[:, :55])          # positions >= 1760 fall past the table row
    lay.block_table = bt
    pool = build_host_pool(w, make_paged_layout(w, 32, seed=5, spare_pages=9, all_pages=True))
    ref_out, ref_lse, _ = oracle.decode_paged_raw(w.q_bits, pool, lay.num_pages, 32, bt, w.idx, w.seqlens,
                                                  w.heads, w.scale, row_format=row_format)
    q = torch.from_numpy(w.q_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    inputs = (q, torch.from_numpy(pool).to(DEV), torch.from_numpy(bt).to(DEV), torch.from_numpy(w.idx).to(DEV),
              torch.from_numpy(w.seqlens).to(DEV))
    for ns in (1, 3):
        out, lse = run_paged(w, lay, inputs, num_splits=ns)
        compare(out, lse, ref_out, ref_lse, label=f"paged missing pages fmt{row_format} ns{ns}")


def test_paged_partials_match_oracle_splits():
    w = make_workload(seed=302, batch=3, heads=32, topk=400, seqlens=[5000, 300, 5000], kv_seq_stride=5000,
                      structure="ragged", q_mult=4.0)
    lay = make_paged_layout(w, 64, seed=6, spare_pages=3)
    pool = build_host_pool(w, lay)
    S = smla.num_splits(w.batch, w.heads, w.topk, 5, 1)
    C = smla.split_size(w.batch, w.heads, w.topk, 5, 1)
    ref_o = np.zeros((3, 32, S, 512))
    ref_l = np.zeros((3, 32, S))
    for i, (lo, hi) in enumerate(oracle.split_bounds(w.topk, S, C)):
        ref_o[:, :, i], ref_l[:, :, i], _ = oracle.decode_paged_raw(
            w.q_bits, pool, lay.num_pages, 64, lay.block_table, w.idx, w.seqlens, w.heads, w.scale,
            idx_offset=lo, idx_cols=hi - lo)
    q, pool_d, bt, idx, sl = device_paged_inputs(w, lay)
    o = torch.full((3, 32, S, 512), float("nan"), device=DEV)
    l = torch.full((3, 32, S), float("nan"), device=DEV)
    smla.sparse_mla_decode_partials_paged(q, pool_d, bt, idx, sl, w.scale, o, l, page_size=64,
                                          num_pages=lay.num_pages, num_splits=5)
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(l[fin] - ref_l[fin]).max() <= 1e-3
    assert np.abs(o - ref_o).max() <= 1e-2 * max(1.0, np.abs(ref_o).max() / 4)
    assert np.linalg.norm(o - ref_o) / np.linalg.norm(ref_o) <= 5e-3


def test_paged_pool_beyond_4gb():
    # the used pages sit past the first 4 GiB of a 4.6 GB pool: 64-bit row
    # addressing through the structured buffer
    w = make_workload(seed=303, batch=4, heads=16, topk=256, seqlen=4096, q_mult=2.0)
    lay = make_paged_layout(w, 64, seed=7)
    total = 112_000                                      # x 64 rows x 640 B = 4.59 GB
    shift = total - lay.num_pages
    lay.block_table = np.where(lay.block_table >= 0, lay.block_table + shift, -1).astype(np.int32)
    lay.num_pages = total
    assert shift * 64 * 640 > 2 ** 32
    cache = build_host_cache(w)
    ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                                            w.scale)
    out, lse = run_paged(w, lay, num_splits=0)
    compare(out, lse, ref_out, ref_lse, label="paged pool > 4 GiB")


def test_paged_graph_replays_match_eager_and_oracle():
    # a captured paged split launch (UE8M0 rows, decode and combine kernels):
    # replays interleaved with eager calls on the same workspace give the eager
    # bits, and the eager result matches the paged oracle
    w = make_workload(seed=302, batch=8, heads=64, topk=512, seqlen=8192, row_format=1)
    lay = make_paged_layout(w, 64, seed=7, spare_pages=5)
    ref_out, ref_lse, _ = oracle.decode_paged_raw(w.q_bits, build_host_pool(w, lay), lay.num_pages, 64,
                                                  lay.block_table, w.idx, w.seqlens, w.heads, w.scale,
                                                  row_format=1)
    q, pool, bt, idx, sl = device_paged_inputs(w, lay)
    ns = 4
    ws = torch.empty(smla.workspace_bytes(w.batch, w.heads, w.topk, ns, 1, 1), dtype=torch.uint8, device=DEV)

    def call(out, lse):
        smla.sparse_mla_decode_paged(q, pool, bt, idx, sl, w.scale, out, lse, page_size=64,
                                     num_pages=lay.num_pages, num_splits=ns, workspace=ws, row_format=1)

    out_e = torch.empty((w.batch, w.heads, 512), dtype=torch.bfloat16, device=DEV)
    lse_e = torch.empty((w.batch, w.heads), device=DEV)
    call(out_e, lse_e)
    torch.cuda.synchronize()
    compare(out_e.float().cpu().numpy().astype(np.float64), lse_e.cpu().numpy().astype(np.float64),
            ref_out, ref_lse, label="paged graph eager")
    ref = (out_e.clone(), lse_e.clone())
    out_g = torch.empty_like(out_e)
    lse_g = torch.empty_like(lse_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(out_g, lse_g)
    torch.cuda.synchronize()
    for r in range(3):
        log(f"case: paged graph replay {r}")
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref[0]) and torch.equal(lse_g, ref[1]), r
        call(out_e, lse_e)          # an eager call on the same workspace in between
        torch.cuda.synchronize()
        assert torch.equal(out_e, ref[0]) and torch.equal(lse_e, ref[1]), r
