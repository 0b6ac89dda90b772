"""Helpers shared by the GPU tests: device copies of a workload, calls through
libsmla.so, and the comparison against the fp64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import sparse_mla_decode_02_amd as smla


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_inputs(w, dev="cuda:0"):
    """q bf16 [B,H,512], cache uint8 [B,S,row bytes] (0xFF except selected rows), idx, seqlens."""
    q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    cache = torch.full((w.batch, w.kv_seq_stride, w.row_bytes), 0xFF, dtype=torch.uint8, device=dev)
    valid = w.valid
    b_i, j_i = np.nonzero(valid)
    if len(b_i):
        flat = torch.from_numpy((b_i.astype(np.int64) * w.kv_seq_stride + w.idx[b_i, j_i]).astype(np.int64)).to(dev)
        rows = torch.from_numpy(np.ascontiguousarray(w.rows[b_i, j_i])).to(dev)
        cache.view(-1, w.row_bytes)[flat] = rows
    idx = torch.from_numpy(w.idx).to(dev)
    seqlens = torch.from_numpy(w.seqlens).to(dev)
    return q, cache, idx, seqlens


def run_decode(w, inputs=None, num_splits=0, poison_workspace=True, idx=None):
    q, cache, idx0, seqlens = inputs if inputs is not None else device_inputs(w)
    idx = idx0 if idx is None else idx
    B, H = w.batch, w.heads
    out = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    need = smla.workspace_bytes(B, H, idx.shape[1], num_splits, w.kv_seq_stride, w.row_format)
    ws = None
    if need:
        ws = torch.full((need,), 0xFF if poison_workspace else 0, dtype=torch.uint8, device=q.device)
    smla.sparse_mla_decode(q, cache, idx, seqlens, w.scale, out, lse, num_splits=num_splits,
                           kv_seq_stride=w.kv_seq_stride, workspace=ws, row_format=w.row_format)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def compare(out, lse, ref_out, ref_lse, *, max_abs=1e-2, rel_l2=5e-3, lse_tol=1e-3, label=""):
    """Tolerances: |err| <= 1e-2 where |ref| < 4; where |ref| >= 4 a bf16 value
    cannot be within 1e-2 of every real number (half its spacing there is
    0.0156), so the result must be one of the two bf16 neighbours of ref
    (|err| <= one bf16 spacing).  Relative L2 over the whole tensor <= 5e-3,
    |lse err| <= 1e-3, and -inf lse exactly where the oracle has it."""
    err = np.abs(out - ref_out)
    big = np.abs(ref_out) >= 4.0
    small_err = err[~big].max() if (~big).any() else 0.0
    big_viol = (err[big] > bf16_ulp(ref_out[big])).sum() if big.any() else 0
    denom = np.linalg.norm(ref_out)
    rl2 = np.linalg.norm(out - ref_out) / denom if denom > 0 else np.linalg.norm(out)
    fin = np.isfinite(ref_lse)
    lse_err = np.abs(lse[fin] - ref_lse[fin]).max() if fin.any() else 0.0
    # the strict figures over every element, reported (not asserted) so that each
    # parity record shows whether elements with |ref| >= 4 also met 1e-2
    strict = float(err.max()) if err.size else 0.0
    big_err = float(err[big].max()) if big.any() else 0.0
    info = dict(label=label, max_abs=float(small_err), rel_l2=float(rl2), lse_err=float(lse_err),
                max_ref=float(np.abs(ref_out).max()) if ref_out.size else 0.0, n_big=int(big.sum()),
                big_viol=int(big_viol), strict_max_abs=strict, max_abs_big=big_err,
                n_over_1e2=int((err > max_abs).sum()))
    log("parity", info)
    assert np.isfinite(out).all(), "non-finite outputs"
    assert small_err <= max_abs, info
    assert big_viol == 0, info
    assert rl2 <= rel_l2, info
    assert lse_err <= lse_tol, info
    assert np.array_equal(np.isneginf(lse), ~fin), info
    return info
