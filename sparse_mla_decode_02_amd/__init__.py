"""Python binding of libsmla.so (sparse MLA decode on AMD gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels
of libsmla.so.  Tensors are torch tensors on the GPU (torch provides device
memory and streams); the functions pass their data pointers and the current
HIP stream through the C ABI declared in include/smla.h.  If the library has
not been built, importing works but every call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmla.so")

SMLA_OK = 0
ROW_FP32_SCALES = 0          # SMLA_ROW_FP32_SCALES: 640-byte rows, fp32 group scales
ROW_UE8M0_SCALES = 1         # SMLA_ROW_UE8M0_SCALES: 584-byte rows, exponent-byte scales
ROW_BYTES_OF_FORMAT = {ROW_FP32_SCALES: 640, ROW_UE8M0_SCALES: 584}
ROW_BYTES = 640
LATENT = 512
NOPE = 448
ROPE = 64

STATUS_NAMES = {
    0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_UNSUPPORTED",
    4: "SMLA_ERR_WORKSPACE", 5: "SMLA_ERR_HIP", 6: "SMLA_ERR_ALIGN", 7: "SMLA_ERR_NO_DEVICE",
    8: "SMLA_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024   # SMLA_NOALLOC_SCRATCH_BYTES

EXPORTS = ("sparse_mla_decode", "sparse_mla_decode_partials", "sparse_mla_combine", "sparse_mla_decode_noalloc",
           "sparse_mla_decode_paged", "sparse_mla_decode_partials_paged", "sparse_mla_decode_per_head",
           "sparse_mla_decode_single_launch", "smla_num_splits_single_launch", "smla_workspace_bytes",
           "smla_num_splits", "smla_split_size", "smla_status_str",
           "smla_debug_validate_enabled", "smla_debug_flags")

# condition bits of the SMLA_DEBUG_VALIDATE input scan (smla.h)
DBG_SEQLEN, DBG_INDEX, DBG_PAGE, DBG_DUPLICATE = 1, 2, 4, 8


class SmlaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("kv_seq_stride", ctypes.c_int64), ("row_format", ctypes.c_int32)]


class SmlaPaged(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


class SmlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsmla.so (built by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        shp = ctypes.POINTER(SmlaShape)
        L.smla_num_splits.argtypes = [shp]
        L.smla_num_splits.restype = i32
        L.smla_split_size.argtypes = [shp]
        L.smla_split_size.restype = i32
        L.sparse_mla_decode_partials.argtypes = [vp, vp, vp, vp, f32, shp, vp, vp, vp]
        L.sparse_mla_decode_partials.restype = ctypes.c_int
        L.smla_workspace_bytes.argtypes = [shp]
        L.smla_workspace_bytes.restype = ctypes.c_size_t
        L.smla_status_str.argtypes = [ctypes.c_int]
        L.smla_status_str.restype = ctypes.c_char_p
        L.sparse_mla_decode.argtypes = [vp, vp, vp, vp, f32, vp, vp, shp, vp, ctypes.c_size_t, vp]
        L.sparse_mla_decode.restype = ctypes.c_int
        L.sparse_mla_decode_noalloc.argtypes = [vp, vp, vp, vp, f32, vp, vp, shp, vp]
        L.sparse_mla_decode_noalloc.restype = ctypes.c_int
        L.sparse_mla_combine.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.sparse_mla_combine.restype = ctypes.c_int
        L.sparse_mla_decode_per_head.argtypes = [vp, vp, vp, vp, f32, vp, vp, shp, vp]
        L.sparse_mla_decode_per_head.restype = ctypes.c_int
        pgd = ctypes.POINTER(SmlaPaged)
        L.sparse_mla_decode_paged.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, shp, pgd, vp, ctypes.c_size_t, vp]
        L.sparse_mla_decode_paged.restype = ctypes.c_int
        L.sparse_mla_decode_partials_paged.argtypes = [vp, vp, vp, vp, vp, f32, shp, pgd, vp, vp, vp]
        L.sparse_mla_decode_partials_paged.restype = ctypes.c_int
        L.sparse_mla_decode_single_launch.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, shp, pgd, vp,
                                                      ctypes.c_size_t, vp, vp]
        L.sparse_mla_decode_single_launch.restype = ctypes.c_int
        L.smla_num_splits_single_launch.argtypes = [shp]
        L.smla_num_splits_single_launch.restype = i32
        L.smla_debug_validate_enabled.argtypes = []
        L.smla_debug_validate_enabled.restype = i32
        L.smla_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
        L.smla_debug_flags.restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().smla_status_str(status).decode()


def _check(status: int):
    if status != SMLA_OK:
        raise SmlaError(status, status_str(status))


def debug_validate_enabled() -> bool:
    """True when SMLA_DEBUG_VALIDATE was set when the library was loaded."""
    return bool(lib().smla_debug_validate_enabled())


def debug_flags(clear: bool = False) -> int:
    """SMLA_DBG_* bits found by the input scans on the current device since the
    load or the last clear; synchronizes the device."""
    v = ctypes.c_uint32(0)
    _check(lib().smla_debug_flags(ctypes.byref(v), 1 if clear else 0))
    return v.value


def make_shape(batch, num_heads, topk, num_splits=0, kv_seq_stride=1, row_format=0) -> SmlaShape:
    return SmlaShape(int(batch), int(num_heads), int(topk), int(num_splits), int(kv_seq_stride),
                     int(row_format))


def num_splits(batch, num_heads, topk, num_splits=0, kv_seq_stride=1, row_format=0) -> int:
    s = make_shape(batch, num_heads, topk, num_splits, kv_seq_stride, row_format)
    return int(lib().smla_num_splits(ctypes.byref(s)))


def num_splits_single_launch(batch, num_heads, topk, num_splits=0, kv_seq_stride=1, row_format=0) -> int:
    shape = make_shape(batch, num_heads, topk, num_splits, kv_seq_stride, row_format)
    return int(lib().smla_num_splits_single_launch(ctypes.byref(shape)))


def split_size(batch, num_heads, topk, num_splits=0, kv_seq_stride=1, row_format=0) -> int:
    s = make_shape(batch, num_heads, topk, num_splits, kv_seq_stride, row_format)
    return int(lib().smla_split_size(ctypes.byref(s)))


def workspace_bytes(batch, num_heads, topk, num_splits=0, kv_seq_stride=1, row_format=0) -> int:
    s = make_shape(batch, num_heads, topk, num_splits, kv_seq_stride, row_format)
    return int(lib().smla_workspace_bytes(ctypes.byref(s)))


def _seq_stride(kv_cache, B, row_format):
    if kv_cache is None:
        return 1
    if kv_cache.dim() == 3:
        return kv_cache.shape[1]
    return kv_cache.numel() // (max(B, 1) * ROW_BYTES_OF_FORMAT.get(row_format, ROW_BYTES))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def sparse_mla_decode(q, kv_cache, topk_idx, seqlens, scale, out, lse, *, num_splits=0,
                      kv_seq_stride=None, workspace=None, stream=None, row_format=0):
    """One decode step through libsmla.so.

    q: bf16 [B,H,512]; kv_cache: uint8 [B, kv_seq_stride, R] (or flat), R =
    640 for row_format 0 (fp32 scales) or 584 for row_format 1 (UE8M0 scales);
    topk_idx: int32 [B,topk]; seqlens: int32 [B]; out: bf16 [B,H,512];
    lse: float32 [B,H]; workspace: uint8 device tensor of at least
    workspace_bytes(...) bytes, allocated here when None.
    """
    import torch
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if kv_seq_stride is None:
        kv_seq_stride = _seq_stride(kv_cache, B, row_format)
    shape = make_shape(B, H, topk, num_splits, kv_seq_stride, row_format)
    L = lib()
    need = int(L.smla_workspace_bytes(ctypes.byref(shape)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.sparse_mla_decode(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(seqlens),
                               ctypes.c_float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape),
                               _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream)))
    return out, lse


def sparse_mla_decode_noalloc(q, kv_cache, topk_idx, seqlens, scale, out, lse, *, num_splits=0,
                              kv_seq_stride=None, stream=None, row_format=0):
    """sparse_mla_decode without a workspace: the split partials use the
    library's fixed per-GPU scratch (SMLA_NOALLOC_SCRATCH_BYTES); nothing is
    allocated.  Calls that overlap on one GPU race."""
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if kv_seq_stride is None:
        kv_seq_stride = _seq_stride(kv_cache, B, row_format)
    shape = make_shape(B, H, topk, num_splits, kv_seq_stride, row_format)
    _check(lib().sparse_mla_decode_noalloc(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(seqlens),
                                           ctypes.c_float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape),
                                           _stream_handle(stream)))
    return out, lse


def sparse_mla_decode_partials(q, kv_cache, topk_idx, seqlens, scale, o_part, lse_part, *,
                               num_splits=0, kv_seq_stride=None, stream=None, row_format=0):
    """Decode kernel only: per-split partials o_part fp32 [B,H,S,512], lse_part fp32 [B,H,S]."""
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if kv_seq_stride is None:
        kv_seq_stride = _seq_stride(kv_cache, B, row_format)
    shape = make_shape(B, H, topk, num_splits, kv_seq_stride, row_format)
    _check(lib().sparse_mla_decode_partials(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(seqlens),
                                            ctypes.c_float(scale), ctypes.byref(shape), _ptr(o_part),
                                            _ptr(lse_part), _stream_handle(stream)))
    return o_part, lse_part


def sparse_mla_combine(o_part, lse_part, out, lse, *, stream=None):
    """Merge split partials o_part fp32 [B,H,S,512], lse_part fp32 [B,H,S]."""
    B, H, S, _ = o_part.shape
    _check(lib().sparse_mla_combine(_ptr(o_part), _ptr(lse_part), B, H, S, _ptr(out), _ptr(lse),
                                    _stream_handle(stream)))
    return out, lse


def sparse_mla_decode_single_launch(q, kv_cache, topk_idx, seqlens, scale, out, lse, *, num_splits=0,
                                    kv_seq_stride=None, block_table=None, page_size=None, num_pages=None,
                                    workspace=None, counters=None, stream=None, row_format=0):
    """sparse_mla_decode (block_table None) or sparse_mla_decode_paged (block_table
    and page_size given) as one kernel launch: the last split of each head block
    merges the partials.  counters: uint32/int32 device tensor of at least
    B * H / 16 elements, zero before its first use (allocated zeroed here when
    None); each completed call leaves it zero.  workspace as for
    sparse_mla_decode."""
    import torch
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    paged = None
    if block_table is not None:
        if num_pages is None:
            num_pages = kv_cache.numel() // (ROW_BYTES_OF_FORMAT.get(row_format, ROW_BYTES) * page_size)
        paged = make_paged(page_size, block_table.shape[1], num_pages)
        kv_seq_stride = 1
    elif kv_seq_stride is None:
        kv_seq_stride = _seq_stride(kv_cache, B, row_format)
    shape = make_shape(B, H, topk, num_splits, kv_seq_stride, row_format)
    L = lib()
    need = int(L.smla_workspace_bytes(ctypes.byref(shape)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if counters is None and need > 0:
        counters = torch.zeros(max(B * (H // 16), 1), dtype=torch.int32, device=q.device)
    if counters is not None:
        assert counters.numel() * counters.element_size() >= 4 * B * (H // 16), "counters: B * H / 16 words"
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.sparse_mla_decode_single_launch(_ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(topk_idx),
                                             _ptr(seqlens), ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                             ctypes.byref(shape), ctypes.byref(paged) if paged is not None else None,
                                             _ptr(workspace), ctypes.c_size_t(ws_bytes), _ptr(counters),
                                             _stream_handle(stream)))
    return out, lse


def make_paged(page_size, pages_per_seq, num_pages) -> SmlaPaged:
    return SmlaPaged(int(page_size), int(pages_per_seq), int(num_pages))


def sparse_mla_decode_paged(q, kv_pool, block_table, topk_idx, seqlens, scale, out, lse, *, page_size,
                            num_pages=None, num_splits=0, workspace=None, stream=None, row_format=0):
    """One decode step over a paged pool through libsmla.so.

    kv_pool: uint8 [num_pages * page_size, R] (or flat), R = 640 / 584 for
    row_format 0 / 1; block_table: int32 [B, pages_per_seq]; the rest as for
    sparse_mla_decode.
    """
    import torch
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if num_pages is None:
        num_pages = kv_pool.numel() // (ROW_BYTES_OF_FORMAT.get(row_format, ROW_BYTES) * page_size)
    shape = make_shape(B, H, topk, num_splits, 1, row_format)
    paged = make_paged(page_size, block_table.shape[1], num_pages)
    L = lib()
    need = int(L.smla_workspace_bytes(ctypes.byref(shape)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L.sparse_mla_decode_paged(_ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(topk_idx), _ptr(seqlens),
                                     ctypes.c_float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape),
                                     ctypes.byref(paged), _ptr(workspace), ctypes.c_size_t(ws_bytes),
                                     _stream_handle(stream)))
    return out, lse


def sparse_mla_decode_partials_paged(q, kv_pool, block_table, topk_idx, seqlens, scale, o_part, lse_part, *,
                                     page_size, num_pages=None, num_splits=0, stream=None, row_format=0):
    """Decode kernel only over a paged pool: split partials as sparse_mla_decode_partials."""
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if num_pages is None:
        num_pages = kv_pool.numel() // (ROW_BYTES_OF_FORMAT.get(row_format, ROW_BYTES) * page_size)
    shape = make_shape(B, H, topk, num_splits, 1, row_format)
    paged = make_paged(page_size, block_table.shape[1], num_pages)
    _check(lib().sparse_mla_decode_partials_paged(_ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(topk_idx),
                                                  _ptr(seqlens), ctypes.c_float(scale), ctypes.byref(shape),
                                                  ctypes.byref(paged), _ptr(o_part), _ptr(lse_part),
                                                  _stream_handle(stream)))
    return o_part, lse_part


def sparse_mla_decode_per_head(q, kv_cache, topk_idx, seqlens, scale, out, lse, *, kv_seq_stride=None,
                               stream=None, row_format=0):
    """The per-head SIMT ablation kernel (one wave per (sequence, head), rows
    re-read per head); arguments as for sparse_mla_decode."""
    B, H, _ = q.shape
    topk = topk_idx.shape[1] if topk_idx.dim() == 2 else 0
    if kv_seq_stride is None:
        kv_seq_stride = _seq_stride(kv_cache, B, row_format)
    shape = make_shape(B, H, topk, 0, kv_seq_stride, row_format)
    _check(lib().sparse_mla_decode_per_head(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(seqlens),
                                            ctypes.c_float(scale), _ptr(out), _ptr(lse), ctypes.byref(shape),
                                            _stream_handle(stream)))
    return out, lse
