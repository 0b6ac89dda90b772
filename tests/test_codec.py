"""Pins of the value codecs: fp8 e4m3fn and bf16 decoding in the oracle, and
the generator's encoders, against independent library conversions and the
fixed values of the OCP 8-bit floating point format."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, encode_e4m3fn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_value(code):
    return torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()


def test_e4m3fn_all_codes_match_torch():
    # exhaustive: the oracle's closed-form decoder vs PyTorch's float8_e4m3fn
    for c in range(256):
        ref = torch_e4m3_value(c)
        got = oracle.e4m3fn_value(c)
        if np.isnan(ref):
            assert np.isnan(got), c
        else:
            assert got == ref, (c, got, ref)
            assert np.signbit(got) == np.signbit(ref), c


def test_e4m3fn_format_landmarks():
    # fixed points of the OCP e4m3fn format (largest finite 448, which is why
    # the group scale is amax/448), stored with their source in tests/golden
    with open(os.path.join(GOLDEN, "e4m3fn_landmarks.json")) as f:
        fx = json.load(f)
    for code_hex, val in fx["values"].items():
        got = oracle.e4m3fn_value(int(code_hex, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), code_hex
    finite = [oracle.e4m3fn_value(c) for c in range(256) if not np.isnan(oracle.e4m3fn_value(c))]
    assert max(finite) == 448.0 and min(finite) == -448.0
    assert sum(np.isnan(oracle.e4m3fn_value(c)) for c in range(256)) == 2   # 0x7f, 0xff


def test_e4m3fn_monotone_and_spacing():
    # positive codes 0..0x7e are strictly increasing; spacing doubles per binade
    vals = [oracle.e4m3fn_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    assert vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6     # smallest subnormal / normal


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b, r in zip(bits, ref):
        got = oracle.lib().oracle_bf16_value(int(b))
        assert (np.isnan(r) and np.isnan(got)) or got == r


def test_encoder_matches_torch_cast():
    # generator's fp8 encoder vs torch's fp32 -> float8_e4m3fn cast (RNE)
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 100,
        rng.standard_normal(20000).astype(np.float32) * 0.01,
        rng.uniform(-448, 448, 20000).astype(np.float32),
    ])
    # exact midpoints between neighbouring codes (ties go to even)
    pos = np.array([oracle.e4m3fn_value(c) for c in range(0x7F)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = encode_e4m3fn(x)
    # -0.0 vs +0.0 is the only permitted difference (both decode to zero)
    diff = got != ref
    assert np.all((got[diff] & 0x7F) == 0) and np.all((ref[diff] & 0x7F) == 0)


def test_encoder_saturates_and_nan():
    got = encode_e4m3fn(np.array([448.0, 464.0, 500.0, 1e9, -1e9, np.nan], dtype=np.float32))
    assert list(got[:5]) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert got[5] == 0x7F


def test_quantiser_error_bound():
    # |x/s - dec(code)| <= half a quantum: 2^-4 |dec| for normal codes, 2^-10 for subnormals
    rng = np.random.default_rng(1)
    v = rng.uniform(-448, 448, 50000).astype(np.float32)
    v = np.concatenate([v, rng.uniform(-0.02, 0.02, 5000).astype(np.float32)])
    codes = encode_e4m3fn(v)
    dec = np.array([oracle.e4m3fn_value(c) for c in codes])
    err = np.abs(v.astype(np.float64) - dec)
    normal = np.abs(dec) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(dec[normal]) + 1e-300)
    assert np.all(err[~normal] <= 2.0 ** -10)


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * 10).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(x), ref)
