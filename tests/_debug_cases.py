"""Seeded inputs with planted conditions for the SMLA_DEBUG_VALIDATE input
scan, built the same way by the GPU test and by the child process it starts
(the scan is switched on by the environment when the library loads, so it runs
in a process of its own).  Also the scan's expected result, written from the
condition list in include/smla.h."""

from __future__ import annotations

import numpy as np

from workloads import make_paged_layout, make_workload

PAGE = 32


def _base(seed, topk=100, batch=4, seqlen=500):
    return make_workload(seed=seed, batch=batch, heads=16, topk=topk, seqlen=seqlen, q_mult=2.0)


def _duplicate(w, b, j_from, j_to):
    """Entry j_to repeats entry j_from of list b, with the same row bytes."""
    w.idx[b, j_to] = w.idx[b, j_from]
    w.rows[b, j_to] = w.rows[b, j_from]


def cases():
    """[(name, kind, workload, paged layout or None)]; kind is "decode",
    "paged" or "per_head"."""
    out = []
    out.append(("clean", "decode", _base(401), None))
    w = _base(402)
    w.seqlens[1] = w.kv_seq_stride + 9
    out.append(("seqlen_past_stride", "decode", w, None))
    w = _base(403)
    w.seqlens[2] = -3
    out.append(("seqlen_negative", "decode", w, None))
    w = _base(404)
    w.idx[0, 7] = -5
    out.append(("entry_below_minus_one", "decode", w, None))
    w = _base(405)
    w.idx[3, 50] = w.seqlens[3]
    out.append(("entry_at_seqlen", "decode", w, None))
    w = _base(406, topk=1500, seqlen=4000)      # the repeat is 1395 entries away: two staging rounds
    _duplicate(w, 2, 5, 1400)
    out.append(("duplicate_far", "decode", w, None))
    w = _base(407, topk=300, seqlen=200)        # lists padded with many -1: not a repeat
    out.append(("padding_only", "decode", w, None))
    w = _base(408)
    _duplicate(w, 1, 10, 11)
    out.append(("duplicate_per_head", "per_head", w, None))
    w = _base(409, seqlen=2000)
    lay = make_paged_layout(w, PAGE, seed=11, spare_pages=3)
    out.append(("paged_clean", "paged", w, lay))
    w = _base(410, seqlen=2000)
    lay = make_paged_layout(w, PAGE, seed=12, spare_pages=3)
    lay.block_table[0, int(w.idx[0, 0]) // PAGE] = -1
    out.append(("paged_slot_unset", "paged", w, lay))
    w = _base(411, seqlen=2000)
    lay = make_paged_layout(w, PAGE, seed=13, spare_pages=3)
    lay.block_table[3, int(w.idx[3, 4]) // PAGE] = lay.num_pages + 2
    out.append(("paged_slot_past_pool", "paged", w, lay))
    return out


def expected_flags(w, lay=None) -> int:
    """SMLA_DBG_* bits the scan must report for these inputs."""
    if lay is None:
        reach = w.kv_seq_stride
    else:
        reach = lay.pages_per_seq * lay.page_size
    f = 0
    for b in range(w.batch):
        sl = int(w.seqlens[b])
        if sl < 0 or sl > reach:
            f |= 1
        kept_below = min(max(sl, 0), reach)
        row = w.idx[b].astype(np.int64)
        if ((row < -1) | ((row >= 0) & (row >= sl))).any():
            f |= 2
        kept = row[(row >= 0) & (row < kept_below)]
        if lay is not None and len(kept):
            pg = lay.block_table[b, kept // lay.page_size]
            if ((pg < 0) | (pg >= lay.num_pages)).any():
                f |= 4
        if len(np.unique(kept)) < len(kept):
            f |= 8
    return f
