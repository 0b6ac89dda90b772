"""GPU parity: libsmla.so (through its C ABI) against the fp64 CPU oracle on
the same seeded inputs.  Marked ``gpu``."""

import functools
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_decode_02_amd as smla
from tests._gpu import compare, device_inputs, log, run_decode
from workloads import build_host_cache, config_workload, make_workload

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@functools.lru_cache(maxsize=2)
def cfg_case(n):
    log(f"building workload config {n}")
    w = config_workload(n)
    cache = build_host_cache(w)
    out, lse, used = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens,
                                       w.heads, w.scale)
    del cache
    log(f"oracle config {n}: {used} threads")
    return w, out, lse


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    cfg_case.cache_clear()


def case_small(seed, **kw):
    w = make_workload(seed=seed, **kw)
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale)
    return w, out, lse


# A contiguous cache with fp32 group scales takes the pipelined kernel at every
# split length; the four-wave kernel runs the same long lists in
# test_four_wave_kernel_on_long_contiguous_lists (and the UE8M0 and paged ones
# by default).
CFG_SPLITS = [(1, 1), (1, 2), (1, 0), (2, 4), (2, 0), (3, 1), (3, 2), (3, 4), (3, 0),
              (4, 4), (4, 8), (4, 0), (5, 0), (5, 3), (5, 4), (5, 1)]


@pytest.mark.parametrize("cfg,nsplit", CFG_SPLITS)
def test_config_parity(cfg, nsplit):
    log(f"case: config {cfg} num_splits {nsplit}")
    w, ref_out, ref_lse = cfg_case(cfg)
    out, lse = run_decode(w, num_splits=nsplit)
    compare(out, lse, ref_out, ref_lse, label=f"cfg{cfg}/ns{nsplit}->{smla.num_splits(w.batch, w.heads, w.topk, nsplit)}")


def test_four_wave_kernel_on_long_contiguous_lists(tmp_path):
    # workloads 4 (two splits of 1024 entries) and 5 (one split) through the
    # four-wave kernel, forced by SMLA_KERNEL in a child process
    path = tmp_path / "four_wave.npz"
    env = dict(os.environ, SMLA_KERNEL="four-wave", PYTHONPATH=ROOT)
    log("starting the four-wave child process")
    r = subprocess.run([sys.executable, "-u", "-m", "tests._kernel_child", str(path)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    log(r.stdout[-2000:])
    assert r.returncode == 0, r.stderr[-3000:]
    got = np.load(path)
    for cfg in (4, 5):
        w, ref_out, ref_lse = cfg_case(cfg)
        compare(got[f"cfg{cfg}.out"], got[f"cfg{cfg}.lse"], ref_out, ref_lse, label=f"four-wave cfg{cfg}")


@pytest.mark.parametrize("heads", [16, 32, 48, 64, 128])
@pytest.mark.parametrize("topk,nsplit", [(45, 1), (45, 2), (100, 0), (1, 1)])
def test_head_counts_and_ragged_lists(heads, topk, nsplit):
    log(f"case: heads {heads} topk {topk} nsplit {nsplit}")
    w, ref_out, ref_lse = case_small(100 + heads + topk, batch=3, heads=heads, topk=topk,
                                     seqlens=[300, 50, 7], kv_seq_stride=300, structure="ragged",
                                     q_mult=2.0)
    out, lse = run_decode(w, num_splits=nsplit)
    compare(out, lse, ref_out, ref_lse, label=f"H{heads}/k{topk}/ns{nsplit}")


def test_masked_entries_anywhere_and_out_of_range():
    w = make_workload(seed=7, batch=4, heads=64, topk=128, seqlen=1000)
    rng = np.random.default_rng(7)
    pos = rng.random(w.idx.shape) < 0.3
    w.idx[pos] = -1
    w.idx[rng.random(w.idx.shape) < 0.05] = 1000 + 5     # beyond seqlen (and past the rows)
    w.idx[0, :] = -1                                      # one list with nothing kept
    cache = build_host_cache(w)
    ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale)
    for ns in (1, 2, 4):
        out, lse = run_decode(w, num_splits=ns)
        compare(out, lse, ref_out, ref_lse, label=f"masked/ns{ns}")
        assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_order_of_list_does_not_matter():
    w, ref_out, ref_lse = case_small(8, batch=2, heads=64, topk=256, seqlen=4096, q_mult=4.0)
    inputs = device_inputs(w)
    out1, lse1 = run_decode(w, inputs, num_splits=2)
    srt = torch.from_numpy(np.sort(w.idx, axis=1)).to("cuda:0")
    out2, lse2 = run_decode(w, inputs, num_splits=2, idx=srt)
    compare(out1, lse1, ref_out, ref_lse, label="shuffled")
    compare(out2, lse2, ref_out, ref_lse, label="sorted")


def test_deterministic_across_runs():
    w, _, _ = case_small(9, batch=8, heads=64, topk=512, seqlen=8192)
    inputs = device_inputs(w)
    a = run_decode(w, inputs, num_splits=4)
    b = run_decode(w, inputs, num_splits=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_single_token_returns_row_exactly():
    # one kept entry with unit scales: out is the row itself in bf16 (fp8 codes
    # are exact in bf16; the device fp8 decode sees every non-NaN code)
    w = make_workload(seed=10, batch=1, heads=16, topk=8, seqlen=4)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = w.rows[0, 0].copy()
    row[:448] = np.resize(codes, 448)
    row[448:476] = np.ones(7, dtype=np.float32).view(np.uint8)
    w.rows[0, :] = row
    w.idx[0] = [2, -1, -1, -1, -1, -1, -1, -1]
    w.q_bits[:] = 0
    cache = build_host_cache(w)
    ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale)
    for ns in (1, 2):
        out, lse = run_decode(w, num_splits=ns)
        assert np.array_equal(out, ref_out), ns      # exact: every value is a bf16 number
        assert np.all(lse == 0.0)


def test_device_fp8_decode_in_logits():
    # q = e_i selects one nope column: lse = scale * e4m3(code_i) (single kept row)
    w = make_workload(seed=12, batch=16, heads=16, topk=1, seqlen=1)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = w.rows[0, 0].copy()
    row[:448] = np.resize(codes, 448)
    row[448:476] = np.ones(7, dtype=np.float32).view(np.uint8)
    w.rows[:, 0] = row
    w.idx[:] = 0
    q = np.zeros((16, 16, 512), dtype=np.uint16)
    cols = np.arange(256).reshape(16, 16) % 448
    for b in range(16):
        for h in range(16):
            q[b, h, cols[b, h]] = 0x3F80     # bf16 1.0
    w.q_bits = q
    out, lse = run_decode(w, num_splits=1)
    expect = np.array([[w.scale * oracle.e4m3fn_value(row[cols[b, h]]) for h in range(16)] for b in range(16)])
    assert np.allclose(lse, expect, rtol=1e-6, atol=1e-7)


def test_empty_batch_and_empty_lists():
    w = make_workload(seed=13, batch=2, heads=16, topk=0, seqlen=10)
    out, lse = run_decode(w, num_splits=0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    w0 = make_workload(seed=14, batch=0, heads=16, topk=8, seqlen=10)
    q = torch.zeros((0, 16, 512), dtype=torch.bfloat16, device="cuda:0")
    out0 = torch.zeros((0, 16, 512), dtype=torch.bfloat16, device="cuda:0")
    smla.sparse_mla_decode(q, torch.zeros((0, 10, 640), dtype=torch.uint8, device="cuda:0"),
                           torch.zeros((0, 8), dtype=torch.int32, device="cuda:0"),
                           torch.zeros((0,), dtype=torch.int32, device="cuda:0"), w0.scale, out0,
                           torch.zeros((0, 16), device="cuda:0"), kv_seq_stride=10)
    torch.cuda.synchronize()


def test_combine_kernel_against_oracle_combine():
    # partials from the oracle (including empty splits) merged by the GPU combine
    w = make_workload(seed=15, batch=3, heads=32, topk=96, seqlens=[40, 500, 2], structure="ragged",
                      kv_seq_stride=500, q_mult=4.0)
    cache = build_host_cache(w)
    o_p, l_p = oracle.decode_splits(w, 5, cache)
    ref_out, ref_lse = oracle.combine(o_p, l_p)
    o_dev = torch.from_numpy(o_p.astype(np.float32)).to("cuda:0")
    l_dev = torch.from_numpy(l_p.astype(np.float32)).to("cuda:0")
    out = torch.empty((3, 32, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((3, 32), dtype=torch.float32, device="cuda:0")
    smla.sparse_mla_combine(o_dev, l_dev, out, lse)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            ref_out, ref_lse, label="combine")


@pytest.mark.parametrize("topk,nsplit", [(512, 4), (200, 3), (96, 8)])
def test_split_partials_against_oracle_partials(topk, nsplit):
    # the decode kernel alone: each split's normalised output and lse
    w = make_workload(seed=16, batch=4, heads=64, topk=topk, seqlens=[3000, 150, 20, 3000],
                      kv_seq_stride=3000, structure="ragged", q_mult=4.0)
    S = smla.num_splits(w.batch, w.heads, w.topk, nsplit, w.kv_seq_stride)
    C = smla.split_size(w.batch, w.heads, w.topk, nsplit, w.kv_seq_stride)
    cache = build_host_cache(w)
    ref_o, ref_l = oracle.decode_splits(w, S, cache, chunk=C)
    q, cache_d, idx, seqlens = device_inputs(w)
    o = torch.full((4, 64, S, 512), float("nan"), device="cuda:0")
    l = torch.full((4, 64, S), float("nan"), device="cuda:0")
    smla.sparse_mla_decode_partials(q, cache_d, idx, seqlens, w.scale, o, l, num_splits=nsplit)
    torch.cuda.synchronize()
    o = o.cpu().numpy().astype(np.float64)
    l = l.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(l[fin] - ref_l[fin]).max() <= 1e-3
    err = np.abs(o - ref_o)
    assert err.max() <= 1e-2 * max(1.0, np.abs(ref_o).max() / 4), err.max()
    assert np.linalg.norm(o - ref_o) / np.linalg.norm(ref_o) <= 5e-3


def test_workspace_reused_across_calls_and_shapes():
    # one workspace, filled with arbitrary bytes once, serves calls of different
    # shapes and split counts in a row
    wa, ra_out, ra_lse = case_small(17, batch=6, heads=32, topk=300, seqlen=4000)
    wb, rb_out, rb_lse = case_small(18, batch=3, heads=64, topk=512, seqlen=2048)
    ia, ib = device_inputs(wa), device_inputs(wb)
    need = max(smla.workspace_bytes(wa.batch, wa.heads, wa.topk, 5, wa.kv_seq_stride),
               smla.workspace_bytes(wb.batch, wb.heads, wb.topk, 3, wb.kv_seq_stride))
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda:0")
    for w, inp, ns, r_out, r_lse, tag in [(wa, ia, 5, ra_out, ra_lse, "a5"), (wb, ib, 3, rb_out, rb_lse, "b3"),
                                          (wa, ia, 2, ra_out, ra_lse, "a2"), (wa, ia, 5, ra_out, ra_lse, "a5'")]:
        log(f"case: workspace reuse {tag}")
        q, cache, idx, sl = inp
        out = torch.full((w.batch, w.heads, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.full((w.batch, w.heads), float("nan"), device="cuda:0")
        smla.sparse_mla_decode(q, cache, idx, sl, w.scale, out, lse, num_splits=ns,
                               kv_seq_stride=w.kv_seq_stride, workspace=ws)
        torch.cuda.synchronize()
        compare(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                r_out, r_lse, label=f"workspace reuse {tag}")


def test_graph_replays_match_eager():
    # a captured split launch (decode and combine kernels); replays interleaved
    # with eager calls on the same workspace must all give the eager result
    w, _, _ = case_small(19, batch=8, heads=64, topk=512, seqlen=8192)
    q, cache, idx, sl = device_inputs(w)
    ns = 4
    ws = torch.empty(smla.workspace_bytes(w.batch, w.heads, w.topk, ns, w.kv_seq_stride),
                     dtype=torch.uint8, device="cuda:0")
    out_e = torch.empty((w.batch, w.heads, 512), dtype=torch.bfloat16, device="cuda:0")
    lse_e = torch.empty((w.batch, w.heads), device="cuda:0")
    smla.sparse_mla_decode(q, cache, idx, sl, w.scale, out_e, lse_e, num_splits=ns,
                           kv_seq_stride=w.kv_seq_stride, workspace=ws)
    torch.cuda.synchronize()
    ref = (out_e.clone(), lse_e.clone())
    out_g = torch.empty_like(out_e)
    lse_g = torch.empty_like(lse_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            smla.sparse_mla_decode(q, cache, idx, sl, w.scale, out_g, lse_g, num_splits=ns,
                                   kv_seq_stride=w.kv_seq_stride, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        log(f"case: graph replay {r}")
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref[0]) and torch.equal(lse_g, ref[1]), r
        if r % 2 == 0:   # an eager call on the same workspace in between
            smla.sparse_mla_decode(q, cache, idx, sl, w.scale, out_e, lse_e, num_splits=ns,
                                   kv_seq_stride=w.kv_seq_stride, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out_e, ref[0]) and torch.equal(lse_e, ref[1]), r


@pytest.mark.parametrize("batch,heads,nsplit", [(5, 16, 7), (3, 48, 5)])
def test_many_splits_on_grids_without_xcd_remap(batch, heads, nsplit):
    # grids that are not a multiple of 8 keep the hardware's round-robin
    # placement of workgroups on XCDs
    w, ref_out, ref_lse = case_small(20 + batch, batch=batch, heads=heads, topk=1024, seqlen=6000)
    grid = batch * (heads // 16) * smla.num_splits(batch, heads, 1024, nsplit, w.kv_seq_stride)
    assert grid % 8 != 0
    inputs = device_inputs(w)
    for rep in range(2):
        log(f"case: splits without remap B={batch} H={heads} ns={nsplit} rep {rep}")
        out, lse = run_decode(w, inputs, num_splits=nsplit)
        compare(out, lse, ref_out, ref_lse, label=f"no-remap B{batch} H{heads} ns{nsplit} #{rep}")
