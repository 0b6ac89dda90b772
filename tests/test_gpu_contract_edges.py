"""GPU parity at the edges of the numerical contract in smla.h: group scales
near the top of the accepted range (fp16 weights p * scale up to 2^8 * 255),
and scales small enough that the fp16 weights are subnormal or underflow,
in both row formats, over many rows and every split count.  The oracle reads
the same bytes, so the comparison is exact up to the kernel's rounding.

Rows with large scales hold values up to 448 * 255, so an output element can
be small only by cancellation among large terms, and the 1e-2 absolute bar
of the benchmark workloads (values of order 1) does not apply to it.  Those
cases are held to the bound the arithmetic gives instead: an fp16 weight
errs by at most 2^-11 of itself, so an element errs by at most 2^-11 times
the largest |V| of its column among the sequence's kept rows (taken here
with a factor 2 for the fp32 sums), plus the bf16 rounding of the result
(2^-8 relative at most); relative L2 <= 5e-3 and |lse error| <= 1e-3 as
everywhere."""

import numpy as np
import pytest
import torch

import oracle
from tests._gpu import compare, log, run_decode
from workloads import build_host_cache, make_workload

pytestmark = pytest.mark.gpu

SCALE_OFF, UE8M0_OFF = 448, 448


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _with_scales(seed, row_format, scales, q_mult):
    """Workload of 4 sequences x 64 heads, top-256 of 2048, whose rows keep the
    generator's codes and rope but carry the given group scales: fp32 values
    [B, topk, 7] (row format 0) or exponent bytes (row format 1)."""
    w = make_workload(seed=seed, batch=4, heads=64, topk=256, seqlen=2048, q_mult=q_mult,
                      row_format=row_format)
    if row_format == 0:
        w.rows[:, :, SCALE_OFF:SCALE_OFF + 28] = np.ascontiguousarray(scales, dtype=np.float32).view(
            np.uint8).reshape(w.batch, w.topk, 28)
    else:
        w.rows[:, :, UE8M0_OFF:UE8M0_OFF + 7] = np.asarray(scales, dtype=np.uint8)
    return w


def _column_vmax(w):
    """max |V[d]| over each sequence's kept rows (oracle dequantisation): [B, 512]."""
    vmax = np.zeros((w.batch, 512))
    for b in range(w.batch):
        for j in np.nonzero(w.valid[b])[0]:
            vmax[b] = np.maximum(vmax[b], np.abs(oracle.dequant_row(w.rows[b, j], w.row_format)))
    return vmax


def _compare_scaled(out, lse, ref_out, ref_lse, vmax, label):
    err = np.abs(out - ref_out)
    bound = 2.0 ** -10 * vmax[:, None, :] + 2.0 ** -8 * np.abs(ref_out) + 1e-6
    rl2 = np.linalg.norm(out - ref_out) / np.linalg.norm(ref_out)
    lse_err = float(np.abs(lse - ref_lse).max())
    info = dict(label=label, worst_err_over_bound=float((err / bound).max()), rel_l2=float(rl2),
                lse_err=lse_err, max_ref=float(np.abs(ref_out).max()), strict_max_abs=float(err.max()))
    log("parity (derived bound)", info)
    assert np.isfinite(out).all() and np.isfinite(lse).all(), info
    assert (err <= bound).all(), info
    assert rl2 <= 5e-3 and lse_err <= 1e-3, info


def _check(w, label, scaled=False):
    cache = build_host_cache(w)
    ref_out, ref_lse, _ = oracle.decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                                            w.scale, row_format=w.row_format)
    vmax = _column_vmax(w) if scaled else None
    for ns in (1, 2, 4, 8, 0):
        log(f"case: {label} num_splits {ns}")
        out, lse = run_decode(w, num_splits=ns)
        if scaled:
            _compare_scaled(out, lse, ref_out, ref_lse, vmax, label=f"{label}/ns{ns}")
        else:
            compare(out, lse, ref_out, ref_lse, label=f"{label}/ns{ns}")


def test_fp32_scales_at_the_top_of_the_range():
    # scales in [128, 255]: values reach 448 * 255; the query is scaled down so
    # that logits stay O(10) (a peaky softmax), and weights p * scale reach
    # ~2^8 * 255, just below the fp16 maximum
    rng = np.random.default_rng(501)
    s = rng.uniform(128.0, 255.0, size=(4, 256, 7)).astype(np.float32)
    s[0, :, :] = 255.0
    w = _with_scales(501, 0, s, q_mult=4.0 * 2.0 ** -14)
    _check(w, "fp32 scales 128..255", scaled=True)


def test_fp32_scales_with_subnormal_fp16_weights():
    # scales in [2^-30, 2^-14]: every nope weight p * scale is an fp16
    # subnormal or underflows to zero; the nope values are then that small too
    rng = np.random.default_rng(502)
    s = np.exp2(rng.uniform(-30.0, -14.0, size=(4, 256, 7))).astype(np.float32)
    w = _with_scales(502, 0, s, q_mult=4.0)
    _check(w, "fp32 scales 2^-30..2^-14")


def test_fp32_scales_spanning_the_whole_range_per_group():
    rng = np.random.default_rng(503)
    s = np.exp2(rng.uniform(-30.0, np.log2(255.0), size=(4, 256, 7))).astype(np.float32)
    w = _with_scales(503, 0, s, q_mult=4.0 * 2.0 ** -12)
    _check(w, "fp32 scales 2^-30..255", scaled=True)


def test_ue8m0_bytes_80_to_110():
    # 2^-47 .. 2^-17: subnormal or underflowing fp16 weights
    rng = np.random.default_rng(504)
    e = rng.integers(80, 110, size=(4, 256, 7), endpoint=True)
    w = _with_scales(504, 1, e, q_mult=4.0)
    _check(w, "ue8m0 bytes 80..110")


def test_ue8m0_bytes_at_the_top_of_the_range():
    # 2^-7 .. 2^7 (byte 134 is the largest the contract accepts)
    rng = np.random.default_rng(505)
    e = rng.integers(120, 134, size=(4, 256, 7), endpoint=True)
    e[1, :, :] = 134
    w = _with_scales(505, 1, e, q_mult=4.0 * 2.0 ** -12)
    _check(w, "ue8m0 bytes 120..134", scaled=True)
