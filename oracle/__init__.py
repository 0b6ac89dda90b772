"""CPU oracle for sparse MLA decode -- TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it; the
two share no code.  Inputs come from the seeded generator in ``workloads``.

* ``oracle.c`` (compiled to ``liboracle.so`` with gcc + OpenMP): the fp64
  plain-definition oracle and its padded-512 twin.
* ``combine()`` here: the fp64 log-sum-exp merge of split partials.
* ``brute.py``: an independent NumPy / PyTorch-CPU dense check for tiny inputs.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build() -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm"],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_value.restype = f64
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = f64
        L.oracle_dequant_row.argtypes = [vp, vp]
        L.oracle_dequant_row.restype = None
        L.oracle_dequant_row_fmt.argtypes = [vp, i32, vp]
        L.oracle_dequant_row_fmt.restype = None
        L.oracle_ue8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_ue8m0_value.restype = f64
        L.oracle_decode.argtypes = [vp, vp, i64, vp, i64, vp, i32, i32, i32, f64, vp, vp, i32]
        L.oracle_decode.restype = i32
        L.oracle_decode_fmt.argtypes = [vp, vp, i64, vp, i64, vp, i32, i32, i32, f64, vp, vp, i32, i32]
        L.oracle_decode_fmt.restype = i32
        L.oracle_decode_paged.argtypes = [vp, vp, i64, i32, vp, i64, vp, i64, vp, i32, i32, i32, f64, vp,
                                          vp, i32, i32]
        L.oracle_decode_paged.restype = i32
        L.oracle_decode_padded512.argtypes = [vp, vp, i64, vp, i64, vp, i32, i32, i32, f64, vp, vp]
        L.oracle_decode_padded512.restype = i32
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def e4m3fn_value(code: int) -> float:
    return lib().oracle_e4m3fn_value(int(code))


ROW_BYTES_OF_FORMAT = {0: 640, 1: 584}


def ue8m0_value(e: int) -> float:
    return lib().oracle_ue8m0_value(int(e))


def dequant_row(row: np.ndarray, row_format: int = 0) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    assert row.shape == (ROW_BYTES_OF_FORMAT[row_format],)
    K = np.empty(512, dtype=np.float64)
    lib().oracle_dequant_row_fmt(_p(row), int(row_format), _p(K))
    return K


def decode_raw(q_bits, cache, kv_seq_stride, idx, seqlens, heads, scale, *, padded512=False,
               nthreads=0, idx_cols=None, idx_offset=0, idx_row_stride=None, row_format=0):
    """out fp64 [B,H,512], lse fp64 [B,H], threads used.

    ``idx`` int32 [B, topk]; the list of sequence b is
    idx[b, idx_offset : idx_offset + idx_cols] (a split of the list).
    ``row_format`` 0: 640-byte rows with fp32 scales; 1: 584-byte rows with
    UE8M0 scales.
    """
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    B = q_bits.shape[0]
    topk = idx.shape[1]
    if idx_cols is None:
        idx_cols = topk - idx_offset
    out = np.zeros((B, heads, 512), dtype=np.float64)
    lse = np.zeros((B, heads), dtype=np.float64)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous
    assert cache.size >= B * kv_seq_stride * ROW_BYTES_OF_FORMAT[row_format]
    idx_view = idx[:, idx_offset:]
    ptr = ctypes.c_void_p(idx.ctypes.data + 4 * idx_offset)
    stride = topk if idx_row_stride is None else idx_row_stride
    if padded512:
        assert row_format == 0
        used = lib().oracle_decode_padded512(_p(q_bits), _p(cache), kv_seq_stride, ptr, stride,
                                             _p(seqlens), B, heads, idx_cols, float(scale),
                                             _p(out), _p(lse))
    else:
        used = lib().oracle_decode_fmt(_p(q_bits), _p(cache), kv_seq_stride, ptr, stride, _p(seqlens),
                                       B, heads, idx_cols, float(scale), _p(out), _p(lse), int(nthreads),
                                       int(row_format))
    del idx_view
    return out, lse, used


def decode_paged_raw(q_bits, pool, num_pages, page_size, block_table, idx, seqlens, heads, scale, *,
                     row_format=0, nthreads=0, idx_offset=0, idx_cols=None):
    """Oracle over a paged pool: ``pool`` uint8 [num_pages * page_size, row bytes],
    ``block_table`` int32 [B, pages_per_seq].  Returns out, lse, threads used."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    B = q_bits.shape[0]
    topk = idx.shape[1]
    if idx_cols is None:
        idx_cols = topk - idx_offset
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    assert pool.size >= num_pages * page_size * ROW_BYTES_OF_FORMAT[row_format]
    assert block_table.shape[0] == B
    out = np.zeros((B, heads, 512), dtype=np.float64)
    lse = np.zeros((B, heads), dtype=np.float64)
    ptr = ctypes.c_void_p(idx.ctypes.data + 4 * idx_offset)
    used = lib().oracle_decode_paged(_p(q_bits), _p(pool), int(num_pages), int(page_size), _p(block_table),
                                     int(block_table.shape[1]), ptr, topk, _p(seqlens), B, heads, idx_cols,
                                     float(scale), _p(out), _p(lse), int(nthreads), int(row_format))
    return out, lse, used


def decode_paged(w, layout, pool=None, **kw):
    """Oracle on a ``workloads.Workload`` stored in the paged ``layout``."""
    if pool is None:
        from workloads import build_host_pool
        pool = build_host_pool(w, layout)
    out, lse, _ = decode_paged_raw(w.q_bits, pool, layout.num_pages, layout.page_size, layout.block_table,
                                   w.idx, w.seqlens, w.heads, w.scale, row_format=w.row_format, **kw)
    return out, lse


def decode(w, cache=None, **kw):
    """Oracle on a ``workloads.Workload``; builds the host cache when not given."""
    if cache is None:
        from workloads import build_host_cache
        cache = build_host_cache(w)
    out, lse, _ = decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                             w.scale, row_format=w.row_format, **kw)
    return out, lse


def split_bounds(topk: int, nsplit: int, chunk: int | None = None):
    """Contiguous chunks of the list: split i covers [i*c, min((i+1)*c, topk)),
    c = ceil(topk / nsplit) unless given."""
    c = chunk if chunk is not None else (-(-topk // nsplit) if topk else 0)
    return [(min(i * c, topk), min((i + 1) * c, topk)) for i in range(nsplit)]


def decode_splits(w, nsplit, cache=None, chunk=None):
    """Per-split partial results: o fp64 [B,H,S,512] (normalised), lse fp64 [B,H,S]."""
    if cache is None:
        from workloads import build_host_cache
        cache = build_host_cache(w)
    o = np.zeros((w.batch, w.heads, nsplit, 512))
    l = np.zeros((w.batch, w.heads, nsplit))
    for i, (lo, hi) in enumerate(split_bounds(w.topk, nsplit, chunk)):
        oi, li, _ = decode_raw(w.q_bits, cache, w.kv_seq_stride, w.idx, w.seqlens, w.heads,
                               w.scale, idx_offset=lo, idx_cols=hi - lo, row_format=w.row_format)
        o[:, :, i] = oi
        l[:, :, i] = li
    return o, l


def combine(o_part: np.ndarray, lse_part: np.ndarray):
    """Log-sum-exp merge of split partials, fp64.

    LSE = M + ln sum_i exp(lse_i - M) with M = max_i lse_i;
    out = sum_i exp(lse_i - LSE) * o_i.  Splits with lse_i = -inf weigh 0;
    when every split is empty, out = 0 and LSE = -inf.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    M = lse_part.max(axis=-1)
    empty = ~np.isfinite(M) & (M < 0)
    Ms = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(lse_part), 0.0, np.exp(lse_part - Ms[..., None]))
    W = w.sum(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(empty[..., None], 0.0,
                       (w[..., None] * o_part).sum(axis=-2) / np.where(empty, 1.0, W)[..., None])
        lse = np.where(empty, -np.inf, Ms + np.log(np.where(empty, 1.0, W)))
    return out, lse
