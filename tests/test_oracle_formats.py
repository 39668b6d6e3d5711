"""Pins of the oracle's element decoders against definitions that do not go
through the oracle: the binary16 closed form, the OCP E4M3 table and torch's
own float8_e4m3fn conversion, and two's complement."""

import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _binary16_closed_form(bits: int) -> float:
    s, e, m = bits >> 15, (bits >> 10) & 0x1F, bits & 0x3FF
    if e == 0x1F:
        return math.nan if m else (-math.inf if s else math.inf)
    mag = (m / 1024.0) * 2.0 ** -14 if e == 0 else (1 + m / 1024.0) * 2.0 ** (e - 15)
    return -mag if s else mag


def test_f16_decode_all_codes_closed_form():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_f16(bits)
    want = np.array([_binary16_closed_form(int(b)) for b in range(65536)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zero survives
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_e4m3fn(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.nanmax(got) == 448.0


def test_e4m3fn_decode_golden_table():
    with open(os.path.join(GOLDEN, "e4m3fn_codes.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code, val in rows:
        got = oracle.decode_e4m3fn(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val), (code, got, val)
            assert math.copysign(1, got) == math.copysign(1, float(val))


def test_int8_decode_twos_complement():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_int8(codes)
    want = np.array([c - 256 if c >= 128 else c for c in range(256)], np.float64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kv", ["fp8_e4m3", "int8"])
def test_dequantize_applies_fp32_scale(kv):
    codes = np.arange(256, dtype=np.uint8)
    sc = np.float32(0.0123)
    got = oracle.dequantize(codes, kv, sc)
    base = oracle.decode_e4m3fn(codes) if kv == "fp8_e4m3" else oracle.decode_int8(codes)
    ok = ~np.isnan(base)
    assert np.array_equal(got[ok], float(sc) * base[ok])
    assert float(sc) == np.float64(sc)  # fp32 widened exactly
