"""Pins of the fp64 CPU oracle against things other than itself: an
independent dense brute-force computation, closed forms, invariants and the
padded-512 formulation of the pages (which must agree bit for bit)."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.brute import brute_decode, dequant_rows_torch, q_values
from workloads import build_host_cache, config_workload, make_workload, quantise_rows, ue8m0_exponents

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(w, **kw):
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                                    w.scale, **kw)
    return out, lse, cache


TINY = [
    dict(seed=11, batch=1, heads=16, topk=16, seqlen=64),
    dict(seed=12, batch=2, heads=16, topk=16, seqlen=40),
    dict(seed=13, batch=2, heads=4 * 4, topk=8, seqlens=[5, 64], structure="ragged"),
    dict(seed=14, batch=2, heads=16, topk=16, seqlen=64, q_mult=4.0),
    dict(seed=15, batch=1, heads=16, topk=16, seqlen=16),
]


@pytest.mark.parametrize("cfg", TINY)
def test_oracle_matches_brute_force(cfg):
    w = make_workload(**cfg)
    out, lse, cache = run(w)
    bout, blse = brute_decode(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.scale)
    scale = max(1.0, np.abs(bout).max())
    assert np.abs(out - bout).max() <= 1e-12 * scale
    fin = np.isfinite(blse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - blse[fin]).max() <= 1e-12 * max(1.0, np.abs(blse[fin]).max())


@pytest.mark.parametrize("cfg", TINY + [dict(seed=21, batch=2, heads=16, topk=64, seqlen=256)])
def test_padded512_formulation_is_bitwise_equal(cfg):
    # columns 448..511 padded with zeros and mapped to the (NaN-filled) pad
    # scale slot, excluded by selection: results must be identical bits
    w = make_workload(**cfg)
    out, lse, cache = run(w)
    sel = cache.reshape(-1, 640)[w.idx[0]]
    assert np.all(np.isnan(sel[:, 476:480].copy().view(np.float32)))   # pad slot holds NaN
    pout, plse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens,
                                      w.heads, w.scale, padded512=True)
    assert np.array_equal(out.view(np.uint64), pout.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), plse.view(np.uint64))


def test_pad_slot_is_never_read():
    # the generator fills scale slot 7 and bytes 608..639 with 0xFF (NaN);
    # any read of them would turn outputs into NaN
    w = make_workload(seed=5, batch=2, heads=16, topk=32, seqlen=128)
    out, lse, cache = run(w)
    rows = cache.reshape(-1, 640)
    used = rows[w.idx[0]]
    assert np.all(used[:, 476:480] == 0xFF) and np.all(used[:, 608:] == 0xFF)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_masked_entries_change_nothing():
    # inserting -1 and out-of-range entries anywhere leaves results bitwise equal
    w = make_workload(seed=31, batch=2, heads=16, topk=24, seqlen=100)
    out, lse, cache = run(w)
    rng = np.random.default_rng(0)
    extra = np.array([[-1, 100, 5000, -7], [-2, 101, -1, 2 ** 30]], dtype=np.int32)
    idx2 = np.concatenate([w.idx, extra], axis=1)
    for b in range(2):
        perm_pos = rng.permutation(idx2.shape[1])
        # keep the valid entries in their original relative order
        valid = [v for v in idx2[b] if 0 <= v < 100]
        junk = [v for v in idx2[b] if not (0 <= v < 100)]
        slots = sorted(perm_pos[:len(junk)])
        row, vi, ji = [], 0, 0
        for pos in range(idx2.shape[1]):
            if ji < len(junk) and pos == slots[ji]:
                row.append(junk[ji]); ji += 1
            else:
                row.append(valid[vi]); vi += 1
        idx2[b] = row
    out2, lse2, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, idx2, w.seqlens, w.heads, w.scale)
    assert np.array_equal(out.view(np.uint64), out2.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), lse2.view(np.uint64))


def test_permutation_invariance():
    w = make_workload(seed=32, batch=2, heads=16, topk=64, seqlen=512, q_mult=4.0)
    out, lse, cache = run(w)
    idx2 = np.ascontiguousarray(np.random.default_rng(1).permuted(w.idx, axis=1))
    out2, lse2, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, idx2, w.seqlens, w.heads, w.scale)
    assert np.abs(out - out2).max() <= 1e-13 * max(1, np.abs(out).max())
    assert np.abs(lse - lse2).max() <= 1e-13 * max(1, np.abs(lse).max())


def test_single_token_returns_its_row():
    w = make_workload(seed=33, batch=2, heads=16, topk=8, seqlens=[1, 300], kv_seq_stride=300)
    w.idx[:] = -1
    w.idx[0, 3] = 0
    w.idx[1, 5] = 123
    out, lse, cache = run(w)
    rows = cache.reshape(2, 300, 640)
    K0 = dequant_rows_torch(rows[0, [0]])[0]
    K1 = dequant_rows_torch(rows[1, [123]])[0]
    q = q_values(w.q_bits)
    assert np.array_equal(out[0], np.broadcast_to(K0, out[0].shape))
    assert np.array_equal(out[1], np.broadcast_to(K1, out[1].shape))
    assert np.allclose(lse[0], w.scale * (q[0] @ K0), rtol=1e-13, atol=1e-13)
    assert np.allclose(lse[1], w.scale * (q[1] @ K1), rtol=1e-13, atol=1e-13)


def test_zero_query_gives_mean_and_log_count():
    w = make_workload(seed=34, batch=2, heads=16, topk=32, seqlens=[20, 200], structure="ragged",
                      kv_seq_stride=200)
    w.q_bits[:] = 0
    out, lse, cache = run(w)
    for b in range(2):
        sel = [t for t in w.idx[b] if 0 <= t < w.seqlens[b]]
        K = dequant_rows_torch(cache.reshape(2, 200, 640)[b, sel])
        assert np.allclose(out[b], K.mean(axis=0)[None], rtol=1e-13, atol=1e-13)
        assert np.allclose(lse[b], np.log(len(sel)), rtol=0, atol=1e-14)


def test_equal_logits_tie():
    # q has only rope components; two rows share their rope but differ in nope:
    # equal logits, so out is the plain mean and lse = z + ln 2
    w = make_workload(seed=35, batch=1, heads=16, topk=2, seqlen=16)
    w.q_bits[:, :, :448] = 0
    cache = build_host_cache(w)
    rows = cache.reshape(16, 640)
    a, b = w.idx[0]
    rows[b, 480:608] = rows[a, 480:608]
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale)
    K = dequant_rows_torch(rows[[a, b]])
    q = q_values(w.q_bits)[0]
    z = w.scale * (q @ K[0])
    assert np.allclose(out[0], ((K[0] + K[1]) / 2)[None], rtol=1e-14, atol=1e-14)
    assert np.allclose(lse[0], z + np.log(2), rtol=1e-14, atol=1e-14)


def test_empty_list():
    w = make_workload(seed=36, batch=2, heads=16, topk=4, seqlens=[0, 10], kv_seq_stride=10)
    w.idx[1] = [-1, 10, 11, -5]
    out, lse, _ = run(w)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_large_scale_limit_selects_argmax_row():
    w = make_workload(seed=37, batch=1, heads=16, topk=16, seqlen=64, scale=1e4)
    out, lse, cache = run(w)
    K = dequant_rows_torch(cache.reshape(64, 640)[w.idx[0]])
    q = q_values(w.q_bits)[0]
    z = q @ K.T
    best = z.argmax(axis=1)
    assert np.allclose(out[0], K[best], rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("nsplit", [1, 2, 3, 4, 7, 16, 40])
def test_split_and_combine_equals_unsplit(nsplit):
    # includes empty splits: the list has 32 entries of which a tail is -1
    w = make_workload(seed=38, batch=2, heads=16, topk=32, seqlens=[12, 400], structure="ragged",
                      kv_seq_stride=400, q_mult=4.0)
    out, lse, cache = run(w)
    o_p, l_p = oracle.decode_splits(w, nsplit, cache)
    cout, clse = oracle.combine(o_p, l_p)
    assert np.abs(cout - out).max() <= 1e-14 * max(1, np.abs(out).max())
    assert np.abs(clse - lse).max() <= 1e-14 * max(1, np.abs(lse).max())


def test_combine_all_empty():
    o = np.random.default_rng(0).standard_normal((2, 3, 4, 512))
    l = np.full((2, 3, 4), -np.inf)
    out, lse = oracle.combine(o, l)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("row_format,name", [(0, "oracle_cfg1.json"), (1, "oracle_cfg1_ue8m0.json")])
def test_golden_regression(row_format, name):
    # values written by tests/golden/make_golden.py from the oracle
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    w = config_workload(1, row_format=row_format)
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                    row_format=row_format)
    assert np.allclose(lse.ravel(), np.array(g["lse"]), rtol=0, atol=1e-12)
    sample = out.reshape(-1)[np.array(g["out_index"])]
    assert np.allclose(sample, np.array(g["out_value"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Row format 1: UE8M0 exponent-byte scales, 584-byte rows
# ---------------------------------------------------------------------------

def run_fmt(w):
    cache = build_host_cache(w)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                                    w.scale, row_format=w.row_format)
    return out, lse, cache


def test_ue8m0_value_landmarks():
    # byte e stands for 2^(e-127); 255 is the NaN encoding
    assert oracle.ue8m0_value(127) == 1.0
    assert oracle.ue8m0_value(128) == 2.0
    assert oracle.ue8m0_value(126) == 0.5
    assert oracle.ue8m0_value(0) == 2.0 ** -127
    assert oracle.ue8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.ue8m0_value(255))


@pytest.mark.parametrize("cfg", TINY)
def test_ue8m0_oracle_matches_brute_force(cfg):
    w = make_workload(row_format=1, **cfg)
    out, lse, cache = run_fmt(w)
    assert cache.shape[-1] == 584
    bout, blse = brute_decode(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.scale,
                              row_format=1)
    scale = max(1.0, np.abs(bout).max())
    assert np.abs(out - bout).max() <= 1e-12 * scale
    fin = np.isfinite(blse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - blse[fin]).max() <= 1e-12 * max(1.0, np.abs(blse[fin]).max())


def _reencode_fp32_scales(rows584: np.ndarray) -> np.ndarray:
    """The same rows in the 640-byte layout, each exponent byte e written as the
    fp32 number 2^(e-127) (exact for e in 1..254)."""
    n = rows584.shape[0]
    e = rows584[:, 448:455].astype(np.int32)
    assert e.min() >= 1 and e.max() <= 254
    s = np.ldexp(np.ones_like(e, dtype=np.float32), e - 127).astype(np.float32)
    r = np.full((n, 640), 0xFF, dtype=np.uint8)
    r[:, :448] = rows584[:, :448]
    r[:, 448:476] = s.view(np.uint8).reshape(n, 28)
    r[:, 480:608] = rows584[:, 456:584]
    return r


@pytest.mark.parametrize("cfg", TINY + [dict(seed=22, batch=2, heads=16, topk=64, seqlen=256,
                                             q_mult=4.0)])
def test_ue8m0_equals_fp32_scale_rows_bitwise(cfg):
    # a UE8M0 row and the same row carrying its scale as an fp32 power of two
    # describe the same numbers: results are identical bits
    w = make_workload(row_format=1, **cfg)
    out, lse, cache = run_fmt(w)
    B, S, _ = cache.shape
    full = np.full((B * S, 640), 0xFF, dtype=np.uint8)
    flat = cache.reshape(B * S, 584)
    used = np.unique(np.concatenate([b * S + w.idx[b][w.valid[b]] for b in range(B)]))
    full[used] = _reencode_fp32_scales(flat[used])
    out0, lse0, _ = oracle.decode_raw(w.q_bits, full.reshape(B, S, 640), w.kv_seq_stride, w.idx,
                                      w.seqlens, w.heads, w.scale)
    assert np.array_equal(out.view(np.uint64), out0.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), lse0.view(np.uint64))


def test_ue8m0_quantiser_scales_are_tight_and_never_saturate():
    rng = np.random.default_rng(7)
    nope = (rng.standard_normal((64, 448)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    nope[3, 64:128] = 0.0                                   # all-zero group -> e = 127
    rows = quantise_rows(nope, np.zeros((64, 64), np.float32), row_format=1)
    e = rows[:, 448:455].astype(np.int64)
    amax = np.abs(nope.reshape(64, 7, 64)).max(axis=2).astype(np.float64)
    s = np.ldexp(1.0, e - 127)
    nz = amax > 0
    assert np.all(amax[nz] / s[nz] <= 448.0)                # no code saturates
    assert np.all(amax[nz] / (s[nz] / 2) > 448.0)           # the next smaller power would
    assert e[3, 1] == 127
    assert np.array_equal(ue8m0_exponents(np.array([448.0, 449.0, 224.0, 0.0])),
                          np.array([127, 128, 126, 127], dtype=np.uint8))


def test_ue8m0_pad_byte_is_never_read():
    w = make_workload(seed=6, batch=2, heads=16, topk=32, seqlen=128, row_format=1)
    out, lse, cache = run_fmt(w)
    used = cache.reshape(-1, 584)[w.idx[0]]
    assert np.all(used[:, 455] == 0xFF)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_ue8m0_dequant_row_matches_brute():
    w = make_workload(seed=8, batch=1, heads=16, topk=16, seqlen=16, row_format=1)
    rows = w.rows.reshape(-1, 584)
    K = dequant_rows_torch(rows, row_format=1)
    for i in range(rows.shape[0]):
        assert np.array_equal(oracle.dequant_row(rows[i], row_format=1), K[i])


# ---------------------------------------------------------------------------
# Paged cache: rows in a shuffled pool of pages, found through a block table
# ---------------------------------------------------------------------------

from oracle.brute import brute_decode_paged  # noqa: E402
from workloads import build_host_pool, make_paged_layout  # noqa: E402

PAGED = [
    (dict(seed=41, batch=3, heads=16, topk=40, seqlens=[100, 7, 300], structure="ragged",
          kv_seq_stride=300), 16),
    (dict(seed=42, batch=2, heads=32, topk=64, seqlen=512, q_mult=4.0), 1),
    (dict(seed=43, batch=2, heads=16, topk=64, seqlen=500), 64),
    (dict(seed=44, batch=2, heads=16, topk=32, seqlen=100), 256),
]


@pytest.mark.parametrize("row_format", [0, 1])
@pytest.mark.parametrize("cfg,page_size", PAGED)
def test_paged_oracle_matches_brute_force(cfg, page_size, row_format):
    w = make_workload(row_format=row_format, **cfg)
    lay = make_paged_layout(w, page_size, seed=cfg["seed"], spare_pages=3)
    pool = build_host_pool(w, lay)
    out, lse = oracle.decode_paged(w, lay, pool)
    bout, blse = brute_decode_paged(w.q_bits, pool, lay.num_pages, page_size, lay.block_table, w.idx,
                                    w.seqlens, w.scale, row_format)
    assert np.abs(out - bout).max() <= 1e-12 * max(1.0, np.abs(bout).max())
    fin = np.isfinite(blse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - blse[fin]).max() <= 1e-12 * max(1.0, np.abs(blse[fin]).max())


@pytest.mark.parametrize("cfg,page_size", PAGED)
def test_paged_equals_contiguous_bitwise(cfg, page_size):
    # the same rows reached through a block table give identical bits
    w = make_workload(**cfg)
    out, lse, _ = run(w)
    lay = make_paged_layout(w, page_size, seed=cfg["seed"] + 1, spare_pages=2, all_pages=True)
    pout, plse = oracle.decode_paged(w, lay)
    assert np.array_equal(out.view(np.uint64), pout.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), plse.view(np.uint64))


def test_paged_page_renaming_is_invariant():
    w = make_workload(seed=45, batch=3, heads=16, topk=48, seqlen=400)
    lay = make_paged_layout(w, 32, seed=1, spare_pages=4)
    pool = build_host_pool(w, lay)
    out, lse = oracle.decode_paged(w, lay, pool)
    perm = np.random.default_rng(2).permutation(lay.num_pages)
    pool2 = np.empty_like(pool).reshape(lay.num_pages, 32, -1)
    pool2[perm] = pool.reshape(lay.num_pages, 32, -1)
    bt2 = np.where(lay.block_table >= 0, perm[np.maximum(lay.block_table, 0)], -1).astype(np.int32)
    out2, lse2, _ = oracle.decode_paged_raw(w.q_bits, pool2.reshape(pool.shape), lay.num_pages, 32, bt2,
                                            w.idx, w.seqlens, w.heads, w.scale)
    assert np.array_equal(out.view(np.uint64), out2.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), lse2.view(np.uint64))


def test_paged_missing_pages_skip_their_entries():
    # a block-table slot that is -1, negative or past the pool, and a position
    # past the table row, each skip the entry: same bits as -1 in the list
    w = make_workload(seed=46, batch=2, heads=16, topk=64, seqlen=512)
    lay = make_paged_layout(w, 16, seed=3, spare_pages=2, all_pages=True)
    pool = build_host_pool(w, lay)
    bt = lay.block_table.copy()
    bt[0, 3], bt[0, 7], bt[1, 5] = -1, -9, lay.num_pages + 4
    short = bt[:, :30]                      # positions >= 480 fall past the table row
    idx2 = w.idx.copy()
    lp = np.where(w.idx >= 0, w.idx, 0) // 16
    drop = ((np.arange(2)[:, None] == 0) & ((lp == 3) | (lp == 7))) | \
           ((np.arange(2)[:, None] == 1) & (lp == 5)) | (lp >= 30)
    assert drop.sum() > 0
    idx2[drop] = -1
    out, lse, _ = oracle.decode_paged_raw(w.q_bits, pool, lay.num_pages, 16, short, w.idx, w.seqlens,
                                          w.heads, w.scale)
    ref, rlse, _ = oracle.decode_paged_raw(w.q_bits, pool, lay.num_pages, 16, lay.block_table, idx2,
                                           w.seqlens, w.heads, w.scale)
    assert np.array_equal(out.view(np.uint64), ref.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), rlse.view(np.uint64))


def test_entries_past_the_stride_are_skipped():
    # seqlens above the stride (a precondition violation) must not reach the
    # next sequence's rows: entries at or past the stride count as masked
    w = make_workload(seed=47, batch=3, heads=16, topk=40, seqlen=200, kv_seq_stride=200)
    cache = build_host_cache(w)
    idx2 = w.idx.copy()
    idx2[:, ::5] = 200 + np.arange(idx2[:, ::5].shape[1])[None, :]
    ref_idx = idx2.copy()
    ref_idx[:, ::5] = -1
    big = np.full(3, 10 ** 6, dtype=np.int32)
    out, lse, _ = oracle.decode_raw(w.q_bits, cache, 200, idx2, big, w.heads, w.scale)
    ref, rlse, _ = oracle.decode_raw(w.q_bits, cache, 200, ref_idx, w.seqlens, w.heads, w.scale)
    assert np.array_equal(out.view(np.uint64), ref.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), rlse.view(np.uint64))


def test_pool_builder_places_only_rows_a_page_holds():
    # entries whose block-table page is unset, negative or past the pool reach
    # no pool row: physical_rows gives -1 for them, the pool builder places the
    # other rows and never indexes outside the pool, and the oracle over that
    # pool equals the oracle with those entries replaced by -1
    from workloads import physical_rows
    w = make_workload(seed=47, batch=3, heads=16, topk=80, seqlen=600)
    lay = make_paged_layout(w, 32, seed=5, spare_pages=2)
    t0 = [int(w.idx[b, 0]) // 32 for b in range(3)]
    lay.block_table[0, t0[0]] = -1
    lay.block_table[1, t0[1]] = -7
    lay.block_table[2, t0[2]] = lay.num_pages + 2
    phys = physical_rows(w, lay)
    pg = np.where(w.idx >= 0, w.idx, 0) // 32
    cut = np.stack([w.valid[b] & (pg[b] == t0[b]) for b in range(3)])
    assert cut.sum() >= 3
    assert (phys[cut] == -1).all()
    assert (phys[w.valid & ~cut] >= 0).all()
    assert phys.max() < lay.num_pages * lay.page_size
    pool = build_host_pool(w, lay)
    out, lse = oracle.decode_paged(w, lay, pool)
    idx2 = np.where(cut, -1, w.idx).astype(np.int32)
    ref, rlse, _ = oracle.decode_paged_raw(w.q_bits, pool, lay.num_pages, 32, lay.block_table, idx2,
                                           w.seqlens, w.heads, w.scale)
    assert np.array_equal(out.view(np.uint64), ref.view(np.uint64))
    assert np.array_equal(lse.view(np.uint64), rlse.view(np.uint64))
