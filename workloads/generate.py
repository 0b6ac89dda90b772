"""Seeded workload generator for sparse MLA decode (inputs only).

Cache row byte layout (one latent KV row of a token, 640-byte stride):

    bytes   0..447  448 "nope" values as fp8 e4m3fn codes (OCP; max 448)
    bytes 448..475  7 fp32 group scales, group g covers nope columns 64g..64g+63
    bytes 476..479  8th scale slot: padding, never read (filled with 0xFF = NaN)
    bytes 480..607  64 "rope" values as bf16
    bytes 608..639  padding (filled with 0xFF)

The 448 + 64 split of the 512-wide latent row, the 7 groups of 64 columns plus
one padding slot, and the fp8 nope / bf16 rope storage follow "The Power-of-Two
Trap" (sections "The Scale Indexing Complication" and "Input Knowledge
Required").  The group scale is amax/448 in fp32, the quantisation used by the
synthetic workloads (the deployed model's power-of-two UE8M0 scales are a
different format).

Row format 1 (UE8M0 scales, 584-byte stride), the deployed model's scale
format ("Input Knowledge Required" of the same page: unsigned 8-bit
exponent-only scales, one per 64-column group):

    bytes   0..447  448 fp8 e4m3fn codes
    bytes 448..454  7 UE8M0 group scales (byte e stands for 2^(e - 127))
    byte  455       8th scale slot: padding (0xFF)
    bytes 456..583  64 rope values as bf16

Its group scale is the smallest power of two s >= amax/448, so no code
saturates.

Every cache row that no top-k entry selects, and every row past a sequence's
length, is 0xFF bytes, which decodes as NaN in fp8, bf16 and fp32: a kernel
that reads a row it should not read produces NaN.

Draw order per workload: seqlens -> idx -> q -> nope -> rope, all from
``numpy.random.Generator(PCG64(seed))``.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

ROW_BYTES = 640
ROW_FMT_FP32 = 0
ROW_FMT_UE8M0 = 1
ROW_BYTES_OF_FORMAT = {ROW_FMT_FP32: 640, ROW_FMT_UE8M0: 584}
UE8M0_SCALE_OFF = 448
UE8M0_ROPE_OFF = 456
NOPE = 448
ROPE = 64
LATENT = NOPE + ROPE
GROUP = 64
NGROUPS = NOPE // GROUP  # 7
SCALE_OFF = 448
ROPE_OFF = 480
FP8_MAX = 448.0


# --------------------------------------------------------------------------
# value encoders (input preparation only)
# --------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """Quantise to OCP fp8 e4m3fn codes: round to nearest even, saturate to +-448.

    e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
    infinities, only S.1111.111 is NaN, so the largest finite value is 448.
    NaN inputs map to 0x7F.
    """
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    sign = np.signbit(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), FP8_MAX)
    _, e = np.frexp(a)                       # a = f * 2**e, f in [0.5, 1)
    exp_unbiased = np.maximum(e - 1, -6)     # subnormals share exponent -6
    quantum = np.ldexp(1.0, exp_unbiased - 3)
    r = np.rint(a / quantum) * quantum       # np.rint: ties to even
    # code from the rounded magnitude r (exactly representable)
    _, er = np.frexp(r)
    er = er - 1
    normal = r >= 2.0 ** -6
    mant_norm = np.where(normal, r / np.ldexp(1.0, er) * 8 - 8, 0)
    code_norm = ((er + 7) << 3) + mant_norm.astype(np.int64)
    code_sub = (r / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_norm, code_sub).astype(np.int64)
    code = np.where(sign, code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def ue8m0_exponents(amax: np.ndarray) -> np.ndarray:
    """Exponent bytes e of the smallest powers of two 2^(e-127) >= amax/448
    (e = 127 when amax is 0), clamped to [1, 254]."""
    r = np.asarray(amax, dtype=np.float64) / FP8_MAX
    f, k = np.frexp(r)                        # r = f * 2**k, f in [0.5, 1)
    up = np.where(f == 0.5, k - 1, k)         # ceil(log2 r)
    e = np.where(r == 0, 127, np.clip(up + 127, 1, 254))
    return e.astype(np.uint8)


def quantise_rows(nope: np.ndarray, rope: np.ndarray, row_format: int = ROW_FMT_FP32) -> np.ndarray:
    """Pack fp32 nope [N,448] and rope [N,64] into cache rows uint8
    [N, row bytes of the format]."""
    nope = np.ascontiguousarray(nope, dtype=np.float32)
    rope = np.ascontiguousarray(rope, dtype=np.float32)
    n = nope.shape[0]
    g = nope.reshape(n, NGROUPS, GROUP)
    amax = np.abs(g).max(axis=2)                                   # [N,7] fp32
    if row_format == ROW_FMT_UE8M0:
        e = ue8m0_exponents(amax)                                  # [N,7]
        scale = np.ldexp(np.float32(1.0), e.astype(np.int32) - 127).astype(np.float32)
        ratio = (g / scale[:, :, None]).astype(np.float32)         # exact: division by 2^k
        codes = encode_e4m3fn(ratio).reshape(n, NOPE)
        rows = np.full((n, ROW_BYTES_OF_FORMAT[ROW_FMT_UE8M0]), 0xFF, dtype=np.uint8)
        rows[:, :NOPE] = codes
        rows[:, UE8M0_SCALE_OFF:UE8M0_SCALE_OFF + NGROUPS] = e
        rows[:, UE8M0_ROPE_OFF:UE8M0_ROPE_OFF + 2 * ROPE] = \
            bf16_bits_from_f32(rope).view(np.uint8).reshape(n, 2 * ROPE)
        return rows
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    ratio = (g / scale[:, :, None]).astype(np.float32)             # fp32 x / s
    codes = encode_e4m3fn(ratio).reshape(n, NOPE)
    rows = np.full((n, ROW_BYTES), 0xFF, dtype=np.uint8)
    rows[:, :NOPE] = codes
    rows[:, SCALE_OFF:SCALE_OFF + 4 * NGROUPS] = scale.view(np.uint8).reshape(n, 4 * NGROUPS)
    rows[:, ROPE_OFF:ROPE_OFF + 2 * ROPE] = bf16_bits_from_f32(rope).view(np.uint8).reshape(n, 2 * ROPE)
    return rows


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    heads: int
    topk: int
    kv_seq_stride: int
    scale: float              # softmax scale (a float32 value)
    seqlens: np.ndarray       # int32 [B]
    idx: np.ndarray           # int32 [B, topk]; -1 = padding
    q_bits: np.ndarray        # uint16 [B, H, 512] bf16 bit patterns
    rows: np.ndarray          # uint8 [B, topk, row bytes]: row of entry (b, j)
    nsplits: tuple = (1,)     # split counts the parity tests use
    row_format: int = ROW_FMT_FP32

    @property
    def row_bytes(self) -> int:
        return ROW_BYTES_OF_FORMAT[self.row_format]

    @property
    def valid(self) -> np.ndarray:
        return (self.idx >= 0) & (self.idx < self.seqlens[:, None])

    @property
    def n_valid_rows(self) -> int:
        return int(self.valid.sum())


def _draw_idx(rng, seqlens, topk, structure):
    B = len(seqlens)
    idx = np.full((B, topk), -1, dtype=np.int32)
    for b in range(B):
        s = int(seqlens[b])
        if structure == "uniform":
            k = min(topk, s)
            idx[b, :k] = rng.choice(s, size=k, replace=False)
        elif structure == "recent20":
            # 20 % of the list inside the last 512 positions, the rest uniform
            # over the earlier positions, all distinct, then shuffled.
            n_recent = int(round(0.2 * topk))
            recent = s - 512 + rng.choice(512, size=n_recent, replace=False)
            early = rng.choice(s - 512, size=topk - n_recent, replace=False)
            row = np.concatenate([recent, early])
            rng.shuffle(row)
            idx[b] = row
        elif structure == "ragged":
            # all positions when the sequence is shorter than top-k, then -1
            if s >= topk:
                idx[b] = rng.choice(s, size=topk, replace=False)
            else:
                idx[b, :s] = rng.permutation(s)
        else:
            raise ValueError(structure)
    return idx


def make_workload(*, name="custom", seed=0, batch, heads, topk, seqlen=None,
                  seqlens=None, kv_seq_stride=None, structure="uniform",
                  q_mult=1.0, scale=None, nsplits=(1,), row_format=ROW_FMT_FP32) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    if seqlens is None:
        seqlens = np.full(batch, seqlen, dtype=np.int32)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    assert seqlens.shape == (batch,)
    if kv_seq_stride is None:
        kv_seq_stride = int(seqlens.max()) if batch else 1
    idx = _draw_idx(rng, seqlens, topk, structure)
    q = rng.standard_normal((batch, heads, LATENT), dtype=np.float32) * np.float32(q_mult)
    nope = rng.standard_normal((batch * topk, NOPE), dtype=np.float32)
    rope = rng.standard_normal((batch * topk, ROPE), dtype=np.float32)
    rows = quantise_rows(nope, rope, row_format).reshape(batch, topk, ROW_BYTES_OF_FORMAT[row_format])
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(LATENT)))
    return Workload(name=name, seed=seed, batch=batch, heads=heads, topk=topk,
                    kv_seq_stride=int(kv_seq_stride), scale=float(np.float32(scale)),
                    seqlens=seqlens, idx=idx, q_bits=bf16_bits_from_f32(q),
                    rows=rows, nsplits=tuple(nsplits), row_format=row_format)


def _cfg5_seqlens(seed):
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    s = rng.integers(1024, 131072, size=64, endpoint=True).astype(np.int32)
    s[0] = 1024      # always exercises the -1 padding
    s[1] = 131072    # always exercises the longest sequence
    return s


# The five synthetic workloads.  Shapes follow the decode setting of the
# pages (one query token per sequence, 16 heads per GPU at TP=4 or all 64).
CONFIGS = {
    1: dict(name="tiny_b1_h16_s256_k64", batch=1, heads=16, topk=64, seqlen=256,
            structure="uniform", nsplits=(1, 2)),
    2: dict(name="b4_h16_s8192_k512", batch=4, heads=16, topk=512, seqlen=8192,
            structure="uniform", nsplits=(4,)),
    3: dict(name="b32_h64_s32768_k512", batch=32, heads=64, topk=512, seqlen=32768,
            structure="uniform", nsplits=(1, 2, 4)),
    4: dict(name="b96_h16_s65536_k2048_recent20", batch=96, heads=16, topk=2048,
            seqlen=65536, structure="recent20", nsplits=(8,)),
    5: dict(name="b64_h64_ragged_k2048_q4", batch=64, heads=64, topk=2048,
            seqlens="cfg5", kv_seq_stride=131072, structure="ragged", q_mult=4.0,
            nsplits=(0,)),
}


def config_workload(cfg: int, row_format: int = ROW_FMT_FP32) -> Workload:
    """Workload number cfg; with row_format 1 the same shapes and draws in the
    UE8M0 row format (its name gets a _ue8m0 suffix)."""
    c = dict(CONFIGS[cfg])
    if c.get("seqlens") == "cfg5":
        c["seqlens"] = _cfg5_seqlens(cfg)
    if row_format == ROW_FMT_UE8M0:
        c["name"] = c["name"] + "_ue8m0"
    return make_workload(seed=cfg, row_format=row_format, **c)


def build_host_cache(w: Workload) -> np.ndarray:
    """Full cache uint8 [B, kv_seq_stride, row bytes]: selected rows placed, rest 0xFF."""
    cache = np.full((w.batch, w.kv_seq_stride, w.row_bytes), 0xFF, dtype=np.uint8)
    v = w.valid
    b_i, j_i = np.nonzero(v)
    cache[b_i, w.idx[b_i, j_i]] = w.rows[b_i, j_i]
    return cache


# --------------------------------------------------------------------------
# paged cache layout (input placement only)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PagedLayout:
    """Rows of every sequence in one pool of pages of ``page_size`` rows:
    ``block_table[b, p]`` is the pool page that holds positions
    p*page_size .. (p+1)*page_size - 1 of sequence b (-1: not allocated)."""
    page_size: int
    num_pages: int
    block_table: np.ndarray   # int32 [B, pages_per_seq]

    @property
    def pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def make_paged_layout(w: Workload, page_size: int, *, seed: int = 0, spare_pages: int = 0,
                      all_pages: bool = False, shuffle: bool = True) -> PagedLayout:
    """Place the workload's rows in a pool.  A logical page gets a pool page
    when a kept list entry falls in it (every page below the sequence length
    with ``all_pages``); the others stay -1.  Pool pages are a random
    permutation (seeded), or in sequence order without ``shuffle``, plus
    ``spare_pages`` pages that no sequence uses."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    pps = max(1, -(-int(w.seqlens.max() if w.batch else 1) // page_size))
    need = np.zeros((w.batch, pps), dtype=bool)
    if all_pages:
        for b in range(w.batch):
            need[b, : -(-int(w.seqlens[b]) // page_size)] = True
    b_i, j_i = np.nonzero(w.valid)
    need[b_i, w.idx[b_i, j_i] // page_size] = True
    n_used = int(need.sum())
    num_pages = n_used + spare_pages
    perm = (rng.permutation(num_pages) if shuffle else np.arange(num_pages)).astype(np.int32)
    bt = np.full((w.batch, pps), -1, dtype=np.int32)
    bt[need] = perm[:n_used]
    return PagedLayout(page_size=int(page_size), num_pages=int(num_pages), block_table=bt)


def physical_rows(w: Workload, layout: PagedLayout) -> np.ndarray:
    """Pool row of every list entry: -1 for an entry that is not kept, or whose
    position lies past its block-table row, or whose page id is outside the
    pool (such an entry reaches no row; it is masked)."""
    ps = layout.page_size
    t = np.where(w.valid, w.idx, 0).astype(np.int64)
    b = np.arange(w.batch)[:, None]
    p = t // ps
    in_table = p < layout.pages_per_seq
    page = layout.block_table[b, np.minimum(p, layout.pages_per_seq - 1)].astype(np.int64)
    ok = w.valid & in_table & (page >= 0) & (page < layout.num_pages)
    return np.where(ok, page * ps + t % ps, -1)


def build_host_pool(w: Workload, layout: PagedLayout) -> np.ndarray:
    """The pool uint8 [num_pages * page_size, row bytes]: kept rows placed, rest 0xFF."""
    pool = np.full((layout.num_pages * layout.page_size, w.row_bytes), 0xFF, dtype=np.uint8)
    phys = physical_rows(w, layout)
    b_i, j_i = np.nonzero(phys >= 0)
    pool[phys[b_i, j_i]] = w.rows[b_i, j_i]
    return pool
