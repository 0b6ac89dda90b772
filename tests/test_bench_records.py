"""bench.py's reading of the committed counter summary (host only): when the
summary was taken on the current kernel source, the bench line's
roofline.traffic must come from it, not silently read as null."""

import re

import pytest

import bench


def test_counter_summary_is_parsed_when_its_digest_matches():
    text = open(bench.COUNTER_SUMMARY).read()
    m = re.search(r"code sha256\[:16\] = ([0-9a-f]{16})", text)
    assert m, "the counter summary names the kernel source it was taken on"
    if m.group(1) != bench.kernel_digest():
        pytest.skip("the kernel source changed since the counters were taken")
    t = bench.counted_traffic(bench.COUNTER_CONFIG, 0)
    assert t is not None and 1e6 < t < 1e9


def test_counter_summary_only_for_its_own_workload():
    assert bench.counted_traffic(bench.COUNTER_CONFIG + 1, 0) is None
    assert bench.counted_traffic(bench.COUNTER_CONFIG, 1) is None


def test_entry_argument_positions_match_the_header():
    # the KV-cold loop of bench.py swaps q, topk_idx and seqlens into prebuilt
    # argument tuples by position: the positions must be those of include/smla.h
    import os
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "smla.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    for name, (qp, ip, sp) in bench.ENTRY_ARG_POS.items():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", hdr)
        assert m, name
        params = [p.strip().split()[-1].lstrip("*") for p in m.group(1).split(",")]
        assert params[qp] == "q", (name, params)
        assert params[ip] == "topk_idx", (name, params)
        assert params[sp] == "seqlens", (name, params)


def test_kernel_digest_follows_the_build_flags(monkeypatch):
    # the profiles' code hash must change with a compiler flag, not only with
    # the kernel sources (a comment edit keeps it)
    from sparse_mla_decode_02_amd import build as hip_build
    d0 = bench.kernel_digest()
    monkeypatch.setattr(hip_build, "SCHED_CLAUSE", [])
    assert bench.kernel_digest() != d0
    monkeypatch.undo()
    assert bench.kernel_digest() == d0
    assert bench.code_digest("int a; // x\n/* y */\n\nint b;") == bench.code_digest("int a;\nint b;")
