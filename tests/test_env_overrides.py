"""The environment overrides of libsmla.so (SMLA_NSPLIT, SMLA_DEBUG_VALIDATE),
read once when the library loads, checked in fresh processes on a machine
without a GPU; and the planted conditions of the debug-scan cases."""

import json
import os
import subprocess
import sys

import pytest

import sparse_mla_decode_02_amd as smla
from tests._debug_cases import cases, expected_flags

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
needs_lib = pytest.mark.skipif(not os.path.exists(smla.LIB_PATH), reason="libsmla.so not built")

PROBE = r"""
import ctypes, json
import sparse_mla_decode_02_amd as smla
v = ctypes.c_uint32(7)
print(json.dumps({
    "validate": int(smla.lib().smla_debug_validate_enabled()),
    "ns_big": smla.num_splits(4, 16, 4096),
    "ns_small": smla.num_splits(4, 16, 64),
    "ns_explicit": smla.num_splits(4, 16, 4096, num_splits=2),
    "ws_big": smla.workspace_bytes(4, 16, 4096),
    "ws_explicit_5": smla.workspace_bytes(4, 16, 4096, num_splits=5),
    "flags_null": smla.lib().smla_debug_flags(None, 0),
    "flags_status": smla.lib().smla_debug_flags(ctypes.byref(v), 1),
    "flags_value": v.value,
}))
"""


def probe(**env):
    e = {k: v for k, v in os.environ.items() if k not in ("SMLA_NSPLIT", "SMLA_DEBUG_VALIDATE")}
    e.update(env)
    e["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, env=e, capture_output=True, text=True,
                       timeout=120, check=True)
    return json.loads(r.stdout.strip().splitlines()[-1])


@needs_lib
def test_defaults_without_overrides():
    d = probe()
    assert d["validate"] == 0
    assert d["ns_explicit"] == 2
    assert d["flags_null"] == 1


@needs_lib
def test_nsplit_override_replaces_the_heuristic_only():
    base = probe()
    d = probe(SMLA_NSPLIT="5")
    assert d["ns_big"] == 5 and d["ws_big"] == d["ws_explicit_5"] > 0
    assert d["ns_small"] == 2           # clamped to the two 32-entry tiles of a 64-entry list
    assert d["ns_explicit"] == 2        # an explicit request is kept
    for bad in ("0", "-3", "abc", "5x", "", "4097"):
        assert probe(SMLA_NSPLIT=bad)["ns_big"] == base["ns_big"], bad


@needs_lib
def test_debug_validate_switch():
    assert probe(SMLA_DEBUG_VALIDATE="1")["validate"] == 1
    assert probe(SMLA_DEBUG_VALIDATE="yes")["validate"] == 1
    assert probe(SMLA_DEBUG_VALIDATE="0")["validate"] == 0
    assert probe(SMLA_DEBUG_VALIDATE="")["validate"] == 0


@needs_lib
def test_debug_flags_errors_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = probe(SMLA_DEBUG_VALIDATE="1")
    assert d["flags_null"] == 1                                   # SMLA_ERR_NULL
    assert d["flags_status"] == 7 and d["flags_value"] == 7       # SMLA_ERR_NO_DEVICE, untouched


PLANTED = {"clean": 0, "seqlen_past_stride": 1, "seqlen_negative": 1 | 2, "entry_below_minus_one": 2,
           "entry_at_seqlen": 2, "duplicate_far": 8, "padding_only": 0, "duplicate_per_head": 8,
           "paged_clean": 0, "paged_slot_unset": 4, "paged_slot_past_pool": 4}


def test_debug_cases_plant_one_condition_each():
    got = {name: expected_flags(w, lay) for name, _, w, lay in cases()}
    assert got == PLANTED
