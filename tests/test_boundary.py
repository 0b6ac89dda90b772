"""The C ABI of libsmla.so on a machine without a GPU: the library loads,
exports every function include/smla.h declares, and rejects bad host-visible
arguments with the documented status before touching any device."""

import ctypes
import os
import re

import pytest

import sparse_mla_decode_02_amd as smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")

needs_lib = pytest.mark.skipif(not os.path.exists(smla.LIB_PATH), reason="libsmla.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_\w+|sparse_mla_\w+)\s*\(", text)))


@needs_lib
def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(smla.EXPORTS)
    L = ctypes.CDLL(smla.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


@needs_lib
def test_status_strings():
    for code in range(9):
        s = smla.status_str(code)
        assert isinstance(s, str) and s
    assert smla.status_str(0) == "ok"
    assert smla.status_str(99) == "unknown status"


@needs_lib
def test_split_resolution_and_workspace_size():
    # one split: no workspace
    assert smla.num_splits(1, 16, 64, num_splits=1) == 1
    assert smla.workspace_bytes(1, 16, 64, num_splits=1) == 0
    # requests are clamped to the number of 32-entry tiles
    assert smla.num_splits(1, 16, 64, num_splits=8) == 2
    assert smla.num_splits(4, 16, 512, num_splits=4) == 4
    assert smla.num_splits(96, 16, 2048, num_splits=8) == 8
    # workspace: fp32 partials [B,H,S,512] then lse [B,H,S], each 256-byte rounded
    rows = 96 * 16 * 8
    up = lambda x: (x + 255) // 256 * 256
    exp = up(rows * 512 * 4) + up(rows * 4)
    assert smla.workspace_bytes(96, 16, 2048, num_splits=8) == exp
    # heuristic always returns a usable count
    for B, H, k in [(1, 16, 64), (32, 64, 512), (64, 64, 2048), (0, 16, 8), (3, 48, 45), (2, 128, 0)]:
        n = smla.num_splits(B, H, k)
        assert n >= 1
        assert n <= max(1, -(-k // 32))
    # the model's picks on the five benchmark workloads (the fastest measured
    # split counts on MI355X): 1, 8, 2, 2, 1
    picks = [smla.num_splits(B, H, k, 0, S) for B, H, k, S in
             [(1, 16, 64, 256), (4, 16, 512, 8192), (32, 64, 512, 32768), (96, 16, 2048, 65536),
              (64, 64, 2048, 131072)]]
    assert picks == [1, 8, 2, 2, 1]
    # invalid shapes
    assert smla.num_splits(1, 15, 64) == -1
    assert smla.num_splits(1, 16, -1) == -1
    assert smla.num_splits(-1, 16, 64) == -1
    assert smla.num_splits(1, 16, 64, kv_seq_stride=0) == -1
    assert smla.workspace_bytes(1, 15, 64) == 0


def _call(L, shape, ptrs=None, ws=None, wsb=0):
    p = ptrs or {}
    fake = ctypes.c_void_p(1 << 20)   # host-side non-null, aligned; never dereferenced
    args = [p.get(n, fake) for n in ("q", "kv", "idx", "seqlens")]
    return L.sparse_mla_decode(*args, ctypes.c_float(0.05), p.get("out", fake), p.get("lse", fake),
                               ctypes.byref(shape) if shape is not None else None,
                               ws, ctypes.c_size_t(wsb), None)


@needs_lib
def test_argument_errors_before_any_device_work():
    L = smla.lib()
    good = smla.make_shape(2, 16, 64, 1, 128)
    assert _call(L, None) == 1                                   # NULL shape
    for n in ("q", "kv", "idx", "seqlens", "out", "lse"):
        assert _call(L, good, {n: None}) == 1, n                  # NULL operand
    assert _call(L, smla.make_shape(2, 20, 64, 1, 128)) == 2      # H not a multiple of 16
    assert _call(L, smla.make_shape(2, 272, 64, 1, 128)) == 2     # H too large
    assert _call(L, smla.make_shape(2, 16, -3, 1, 128)) == 2      # negative topk
    assert _call(L, smla.make_shape(2, 16, (1 << 20) + 1, 1, 128)) == 2   # topk above SMLA_MAX_TOPK
    assert _call(L, smla.make_shape(2, 16, 2 ** 31 - 1, 0, 128)) == 2     # would wrap byte offsets
    assert smla.num_splits(2, 16, (1 << 20) + 1) == -1
    assert smla.num_splits(2, 16, 1 << 20) >= 1                           # the bound itself is valid
    assert _call(L, smla.make_shape(-1, 16, 64, 1, 128)) == 2     # negative batch
    assert _call(L, smla.make_shape(2, 16, 64, -2, 128)) == 2     # negative splits
    assert _call(L, smla.make_shape(2, 16, 64, 1, 0)) == 2        # stride < 1
    assert _call(L, smla.make_shape(2, 16, 64, 1, 128, 2)) == 2   # unknown row format
    assert _call(L, smla.make_shape(2, 16, 64, 1, 128, -1)) == 2
    assert _call(L, good, {"q": ctypes.c_void_p((1 << 20) + 4)}) == 6   # q misaligned
    assert _call(L, good, {"idx": ctypes.c_void_p((1 << 20) + 2)}) == 6  # idx misaligned
    split = smla.make_shape(2, 16, 64, 2, 128)
    need = L.smla_workspace_bytes(ctypes.byref(split))
    assert need > 0
    assert _call(L, split) == 4                                   # workspace missing
    assert _call(L, split, ws=ctypes.c_void_p(1 << 21), wsb=need - 1) == 4
    assert _call(L, split, ws=ctypes.c_void_p((1 << 21) + 16), wsb=need) == 6


@needs_lib
def test_valid_call_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = smla.lib()
    assert _call(L, smla.make_shape(2, 16, 64, 1, 128)) == 7
    assert L.sparse_mla_combine(ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), 1, 16, 2,
                                ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None) == 7
    assert L.sparse_mla_combine(None, ctypes.c_void_p(1 << 20), 1, 16, 2,
                                ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None) == 1
    assert L.sparse_mla_combine(ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), 1, 16, 0,
                                ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None) == 2


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(smla, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(smla, "_lib", None)
    with pytest.raises(RuntimeError, match="HIP library missing"):
        smla.lib()


@needs_lib
def test_row_formats_and_stride_limits():
    # a sequence's rows must stay below 2^31 bytes: the largest stride per format
    for fmt, rb in ((0, 640), (1, 584)):
        top = (2 ** 31 - 1) // rb
        assert smla.num_splits(1, 16, 64, kv_seq_stride=top, row_format=fmt) >= 1
        assert smla.num_splits(1, 16, 64, kv_seq_stride=top + 1, row_format=fmt) == -1
    assert smla.num_splits(1, 16, 64, row_format=2) == -1
    assert smla.workspace_bytes(4, 16, 512, 4, row_format=1) == smla.workspace_bytes(4, 16, 512, 4)


def test_shape_struct_matches_header(tmp_path):
    # the ctypes mirror of smla_shape has the C struct's size and field offsets
    src = tmp_path / "probe.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "smla.h"\n'
        'int main(void) { printf("%zu %zu %zu %zu\\n", sizeof(smla_shape), '
        'offsetof(smla_shape, num_splits), offsetof(smla_shape, kv_seq_stride), '
        'offsetof(smla_shape, row_format)); return 0; }\n')
    exe = tmp_path / "probe"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    S = smla.SmlaShape
    assert [int(x) for x in got] == [ctypes.sizeof(S), S.num_splits.offset, S.kv_seq_stride.offset,
                                     S.row_format.offset]


def _call_paged(L, shape, paged, ptrs=None):
    p = ptrs or {}
    fake = ctypes.c_void_p(1 << 20)
    args = [p.get(n, fake) for n in ("q", "kv", "bt", "idx", "seqlens")]
    return L.sparse_mla_decode_paged(*args, ctypes.c_float(0.05), p.get("out", fake), p.get("lse", fake),
                                     ctypes.byref(shape), ctypes.byref(paged) if paged is not None else None,
                                     None, ctypes.c_size_t(0), None)


@needs_lib
def test_paged_argument_errors_before_any_device_work():
    L = smla.lib()
    good = smla.make_shape(2, 16, 64, 1, 1)
    pg = smla.make_paged(64, 8, 100)
    assert _call_paged(L, good, None) == 1                            # NULL geometry
    assert _call_paged(L, good, pg, {"bt": None}) == 1                # NULL block table
    for bad in (smla.make_paged(48, 8, 100),                          # page size not a power of two
                smla.make_paged(0, 8, 100), smla.make_paged(1 << 21, 8, 100),
                smla.make_paged(64, 0, 100), smla.make_paged(64, 8, 0),
                smla.make_paged(64, 8, (1 << 26))):                  # pool rows reach 2^32
        assert _call_paged(L, good, bad) == 2
    assert _call_paged(L, good, smla.make_paged(64, 8, (1 << 26) - 1)) in (7, 0)   # largest pool: valid
    assert _call_paged(L, good, pg, {"bt": ctypes.c_void_p((1 << 20) + 2)}) == 6   # misaligned table
    assert _call_paged(L, smla.make_shape(2, 16, 64, 1, 1, 3), pg) == 2             # unknown row format
    import torch
    if not torch.cuda.is_available():
        assert _call_paged(L, good, pg) == 7                          # valid, but no device here


@needs_lib
def test_per_head_argument_errors():
    L = smla.lib()
    fake = ctypes.c_void_p(1 << 20)
    good = smla.make_shape(2, 16, 64, 0, 128)

    def call(shape, **over):
        a = dict(q=fake, kv=fake, idx=fake, sl=fake, out=fake, lse=fake)
        a.update(over)
        return L.sparse_mla_decode_per_head(a["q"], a["kv"], a["idx"], a["sl"], ctypes.c_float(0.05), a["out"],
                                            a["lse"], ctypes.byref(shape) if shape is not None else None, None)
    assert call(None) == 1
    assert call(good, out=None) == 1
    assert call(smla.make_shape(2, 20, 64, 0, 128)) == 2
    assert call(good, out=ctypes.c_void_p((1 << 20) + 8)) == 6


@needs_lib
def test_noalloc_argument_errors_before_any_device_work():
    L = smla.lib()
    fake = ctypes.c_void_p(1 << 20)

    def call(shape, **over):
        a = dict(q=fake, kv=fake, idx=fake, sl=fake, out=fake, lse=fake)
        a.update(over)
        return L.sparse_mla_decode_noalloc(a["q"], a["kv"], a["idx"], a["sl"], ctypes.c_float(0.05), a["out"],
                                           a["lse"], ctypes.byref(shape) if shape is not None else None, None)
    assert call(None) == 1                                            # NULL shape
    assert call(smla.make_shape(2, 20, 64, 2, 128)) == 2              # H not a multiple of 16
    # split partials beyond the fixed scratch: rejected before any device work
    big = smla.make_shape(64, 256, 2048, 16, 4096)
    assert L.smla_workspace_bytes(ctypes.byref(big)) > smla.NOALLOC_SCRATCH_BYTES
    assert call(big) == 8
    assert "scratch" in smla.status_str(8)
    # the largest split count that fits at 32 sequences x 64 heads
    fits = smla.make_shape(32, 64, 512, 2, 32768)
    assert 0 < L.smla_workspace_bytes(ctypes.byref(fits)) <= smla.NOALLOC_SCRATCH_BYTES
    import torch
    if not torch.cuda.is_available():
        assert call(fits) == 7                                        # valid, but no device here
        assert call(fits, out=None) in (1, 7)


@needs_lib
def test_single_launch_split_choice():
    # the single launch's model on the five benchmark workloads (its fastest
    # measured split counts on MI355X: 1, 4, 1, 2, 1), never more splits than
    # sparse_mla_decode's (whose workspace it uses), and -1 for invalid shapes
    shapes = [(1, 16, 64, 256), (4, 16, 512, 8192), (32, 64, 512, 32768), (96, 16, 2048, 65536),
              (64, 64, 2048, 131072)]
    assert [smla.num_splits_single_launch(B, H, k, 0, S) for B, H, k, S in shapes] == [1, 4, 1, 2, 1]
    import random
    rng = random.Random(7)
    for _ in range(3000):
        B, H, k = rng.randint(1, 128), 16 * rng.randint(1, 16), rng.randint(1, 8192)
        assert 1 <= smla.num_splits_single_launch(B, H, k, 0, k) <= smla.num_splits(B, H, k, 0, k)
    assert smla.num_splits_single_launch(2, 16, 64, 2, 128) == 2      # a request is kept
    assert smla.num_splits_single_launch(1, 15, 64) == -1


@needs_lib
def test_single_launch_argument_errors():
    L = smla.lib()
    fake = ctypes.c_void_p(1 << 20)

    def call(shape, paged=None, ws=None, wsb=0, **over):
        a = dict(q=fake, kv=fake, bt=fake, idx=fake, sl=fake, out=fake, lse=fake, ctr=ctypes.c_void_p(1 << 22))
        a.update(over)
        return L.sparse_mla_decode_single_launch(
            a["q"], a["kv"], a["bt"], a["idx"], a["sl"], ctypes.c_float(0.05), a["out"], a["lse"],
            ctypes.byref(shape) if shape is not None else None, ctypes.byref(paged) if paged is not None else None,
            ws, ctypes.c_size_t(wsb), a["ctr"], None)
    split = smla.make_shape(2, 16, 64, 2, 128)
    need = L.smla_workspace_bytes(ctypes.byref(split))      # the same split partials as sparse_mla_decode
    assert need > 0
    ws = ctypes.c_void_p(1 << 21)
    assert call(None) == 1                                                  # NULL shape
    assert call(split, ws=ws, wsb=need, out=None) == 1                      # NULL operand
    assert call(smla.make_shape(2, 20, 64, 2, 128)) == 2                    # H not a multiple of 16
    assert call(split, ws=ws, wsb=need, ctr=None) == 1                      # counters missing
    assert call(split, ws=ws, wsb=need, ctr=ctypes.c_void_p((1 << 22) + 2)) == 6   # counters misaligned
    assert call(split) == 4                                                 # workspace missing
    assert call(split, ws=ws, wsb=need - 1) == 4
    assert call(split, ws=ctypes.c_void_p((1 << 21) + 16), wsb=need) == 6   # workspace misaligned
    paged = smla.make_paged(64, 4, 16)
    assert call(split, paged, bt=None, ws=ws, wsb=need) == 1               # no block table
    assert call(split, smla.make_paged(48, 4, 16), ws=ws, wsb=need) == 2    # page size not a power of two
    one = smla.make_shape(2, 16, 64, 1, 128)
    import torch
    if not torch.cuda.is_available():
        assert call(split, ws=ws, wsb=need) == 7                           # valid, but no device here
        assert call(split, paged, ws=ws, wsb=need) == 7
        assert call(one, ctr=None) == 7                                     # one split: no counters needed
