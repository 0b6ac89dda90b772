"""GPU parity of sparse_mla_decode_single_launch (split partials merged by the
last split of each head block inside the decode kernel): bitwise against
sparse_mla_decode with the same split count, and against the fp64 oracle.
Marked ``gpu``."""

import functools

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_decode_02_amd as smla
from tests._gpu import compare, device_inputs, log, run_decode
from workloads import (build_host_cache, config_workload, make_paged_layout, make_workload,
                       physical_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    cfg_case.cache_clear()


@functools.lru_cache(maxsize=1)
def cfg_case(n, row_format):
    log(f"building workload config {n} (row format {row_format}) and its oracle")
    w = config_workload(n, row_format=row_format)
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                    row_format=row_format)
    return w, out, lse


def small_case(seed, **kw):
    w = make_workload(seed=seed, **kw)
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                    row_format=w.row_format)
    return w, out, lse


def run_single(w, inputs, num_splits, ws=None, ctr=None, idx=None):
    q, cache, idx0, sl = inputs
    idx = idx0 if idx is None else idx
    out = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.batch, w.heads), float("nan"), dtype=torch.float32, device=DEV)
    smla.sparse_mla_decode_single_launch(q, cache, idx, sl, w.scale, out, lse, num_splits=num_splits,
                                         kv_seq_stride=w.kv_seq_stride, workspace=ws, counters=ctr,
                                         row_format=w.row_format)
    torch.cuda.synchronize()
    return out, lse


def as_np(out, lse):
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(w, inputs, ns, ref_out, ref_lse, label, ws=None, ctr=None):
    """single launch == sparse_mla_decode with the same resolved split count,
    bit for bit, and within tolerance of the oracle"""
    out, lse = run_single(w, inputs, ns, ws=ws, ctr=ctr)
    res = smla.num_splits_single_launch(w.batch, w.heads, inputs[2].shape[1], ns, w.kv_seq_stride, w.row_format)
    two_out, two_lse = run_decode(w, inputs, num_splits=res)
    o, l = as_np(out, lse)
    assert np.array_equal(o, two_out, equal_nan=True), label
    assert np.array_equal(l, two_lse, equal_nan=True), label
    compare(o, l, ref_out, ref_lse, label=label)


# (workload, row format, split request): the pipelined kernel on every row
# format up to 512 entries per split and on fp32 scales beyond; the four-wave
# kernel on the longer UE8M0 splits; 0 = the single launch's own choice
# (4, 1, 2 and 1 splits at workloads 2, 3, 4 and 5)
CASES = [(2, 0, 0), (3, 0, 0), (3, 0, 2), (3, 0, 4), (3, 1, 2), (4, 0, 0), (4, 1, 2), (5, 0, 3)]


@pytest.mark.parametrize("cfg,row_format,nsplit", CASES)
def test_single_launch_config_parity(cfg, row_format, nsplit):
    log(f"case: single launch config {cfg} row format {row_format} num_splits {nsplit}")
    w, ref_out, ref_lse = cfg_case(cfg, row_format)
    ns = smla.num_splits_single_launch(w.batch, w.heads, w.topk, nsplit, w.kv_seq_stride, row_format)
    assert ns <= smla.num_splits(w.batch, w.heads, w.topk, nsplit, w.kv_seq_stride, row_format)
    check(w, device_inputs(w), nsplit, ref_out, ref_lse, f"single cfg{cfg}/f{row_format}/ns{ns}")


@pytest.mark.parametrize("batch,heads,topk,nsplit", [(5, 48, 100, 3), (3, 16, 45, 2), (1, 128, 700, 7),
                                                      (2, 64, 64, 8)])
def test_single_launch_ragged_shapes(batch, heads, topk, nsplit):
    # grids that are not multiples of 8, a ragged last split, a split request
    # clamped to the tile count
    log(f"case: single launch B={batch} H={heads} topk={topk} ns={nsplit}")
    w, ref_out, ref_lse = small_case(40 + batch, batch=batch, heads=heads, topk=topk, seqlen=3000)
    check(w, device_inputs(w), nsplit, ref_out, ref_lse, f"single B{batch} H{heads} k{topk} ns{nsplit}")


def test_single_launch_with_empty_splits():
    # every entry of the later splits masked: their partials are empty (lse -inf)
    w, _, _ = small_case(47, batch=4, heads=32, topk=256, seqlen=4000)
    idx = w.idx.copy()
    idx[:, 64:] = -1
    idx[1, :] = -1                     # one list keeps nothing at all
    cache = build_host_cache(w)
    ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, idx, w.seqlens, w.heads, w.scale)
    q, cache_d, _, sl = device_inputs(w)
    idx_d = torch.from_numpy(idx).to(DEV)
    out, lse = run_single(w, (q, cache_d, idx_d, sl), 4)
    o, l = as_np(out, lse)
    two_out, two_lse = run_decode(w, (q, cache_d, idx_d, sl), num_splits=4)
    assert np.array_equal(o, two_out) and np.array_equal(l, two_lse)
    assert (o[1] == 0).all() and np.isneginf(l[1]).all()
    compare(o, l, ref_out, ref_lse, label="single empty splits")


def test_single_launch_counters_and_workspace_reused_across_shapes():
    # the arrival counters are left at zero by every call: one counter array
    # and one (poisoned) workspace serve a small call, a large one, another
    # split count, and the small one again
    wa, ra_out, ra_lse = small_case(51, batch=16, heads=64, topk=512, seqlen=8192)
    wb, rb_out, rb_lse = small_case(52, batch=3, heads=32, topk=300, seqlen=2000)
    ia, ib = device_inputs(wa), device_inputs(wb)
    need = smla.workspace_bytes(wa.batch, wa.heads, wa.topk, 4, wa.kv_seq_stride)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    ctr = torch.zeros(wa.batch * wa.heads // 16, dtype=torch.int32, device=DEV)
    for rep, (w, inp, ns, ro, rl) in enumerate([(wb, ib, 3, rb_out, rb_lse), (wa, ia, 4, ra_out, ra_lse),
                                                 (wa, ia, 2, ra_out, ra_lse), (wb, ib, 5, rb_out, rb_lse)]):
        log(f"case: single launch counter reuse call {rep}")
        assert smla.workspace_bytes(w.batch, w.heads, w.topk, ns, w.kv_seq_stride) <= need
        check(w, inp, ns, ro, rl, f"single reuse #{rep}", ws=ws, ctr=ctr)
        torch.cuda.synchronize()
        assert int(ctr.abs().sum()) == 0, rep


def test_single_launch_graph_replays_match_eager():
    w, ref_out, ref_lse = small_case(53, batch=8, heads=64, topk=512, seqlen=8192)
    q, cache, idx, sl = device_inputs(w)
    ns = 4
    ws = torch.empty(smla.workspace_bytes(w.batch, w.heads, w.topk, ns, w.kv_seq_stride),
                     dtype=torch.uint8, device=DEV)
    ctr = torch.zeros(w.batch * w.heads // 16, dtype=torch.int32, device=DEV)
    out_e = torch.empty((w.batch, w.heads, 512), dtype=torch.bfloat16, device=DEV)
    lse_e = torch.empty((w.batch, w.heads), device=DEV)

    def call(out, lse):
        smla.sparse_mla_decode_single_launch(q, cache, idx, sl, w.scale, out, lse, num_splits=ns,
                                             kv_seq_stride=w.kv_seq_stride, workspace=ws, counters=ctr)
    call(out_e, lse_e)
    torch.cuda.synchronize()
    ref = (out_e.clone(), lse_e.clone())
    compare(*as_np(*ref), ref_out, ref_lse, label="single graph eager")
    out_g, lse_g = torch.empty_like(out_e), torch.empty_like(lse_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(out_g, lse_g)
    torch.cuda.synchronize()
    for r in range(4):
        log(f"case: single launch graph replay {r}")
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref[0]) and torch.equal(lse_g, ref[1]), r
        if r % 2 == 0:   # an eager call on the same workspace in between
            call(out_e, lse_e)
            torch.cuda.synchronize()
            assert torch.equal(out_e, ref[0]) and torch.equal(lse_e, ref[1]), r


def device_paged_inputs(w, lay):
    q = torch.from_numpy(w.q_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    pool = torch.full((lay.num_pages * lay.page_size, w.row_bytes), 0xFF, dtype=torch.uint8, device=DEV)
    phys = physical_rows(w, lay)
    b_i, j_i = np.nonzero(phys >= 0)
    assert phys.max(initial=-1) < lay.num_pages * lay.page_size
    if len(b_i):
        pool[torch.from_numpy(phys[b_i, j_i]).to(DEV)] = torch.from_numpy(
            np.ascontiguousarray(w.rows[b_i, j_i])).to(DEV)
    bt = torch.from_numpy(lay.block_table).to(DEV)
    return q, pool, bt, torch.from_numpy(w.idx).to(DEV), torch.from_numpy(w.seqlens).to(DEV)


@pytest.mark.parametrize("cfg,row_format,nsplit", [(3, 1, 2), (4, 1, 2)])
def test_single_launch_paged(cfg, row_format, nsplit):
    # the deployed layout (UE8M0 rows in a pool of 64-row pages): the pipelined
    # kernel's paged instance at workload 3, the four-wave one at workload 4;
    # bitwise equal to sparse_mla_decode_paged, and the oracle on the same rows
    log(f"case: single launch paged config {cfg} row format {row_format} num_splits {nsplit}")
    w, ref_out, ref_lse = cfg_case(cfg, row_format)
    lay = make_paged_layout(w, 64, seed=cfg + 64, spare_pages=7)
    q, pool, bt, idx, sl = device_paged_inputs(w, lay)
    out = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.batch, w.heads), float("nan"), dtype=torch.float32, device=DEV)
    smla.sparse_mla_decode_single_launch(q, pool, idx, sl, w.scale, out, lse, num_splits=nsplit,
                                         block_table=bt, page_size=64, num_pages=lay.num_pages,
                                         row_format=row_format)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    smla.sparse_mla_decode_paged(q, pool, bt, idx, sl, w.scale, out2, lse2, page_size=64,
                                 num_pages=lay.num_pages, num_splits=nsplit, row_format=row_format)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    compare(*as_np(out, lse), ref_out, ref_lse, label=f"single paged cfg{cfg}/f{row_format}")


def test_single_launch_one_split_is_the_plain_launch():
    w, ref_out, ref_lse = small_case(55, batch=4, heads=16, topk=200, seqlen=1000)
    assert smla.workspace_bytes(w.batch, w.heads, w.topk, 1, w.kv_seq_stride) == 0
    check(w, device_inputs(w), 1, ref_out, ref_lse, "single ns1")


def test_single_launch_many_splits_and_heads():
    # 256 heads (16 head blocks, 16 counters per sequence) and 32 splits of a
    # 4096-entry list: the merging workgroup folds in eight groups of four
    w, ref_out, ref_lse = small_case(57, batch=2, heads=256, topk=4096, seqlen=5000)
    assert smla.num_splits_single_launch(w.batch, w.heads, w.topk, 32, w.kv_seq_stride) == 32
    inputs = device_inputs(w)
    ctr = torch.zeros(w.batch * w.heads // 16, dtype=torch.int32, device=DEV)
    for rep in range(2):
        log(f"case: single launch 256 heads 32 splits #{rep}")
        check(w, inputs, 32, ref_out, ref_lse, f"single H256 ns32 #{rep}", ctr=ctr)
        torch.cuda.synchronize()
        assert int(ctr.abs().sum()) == 0
