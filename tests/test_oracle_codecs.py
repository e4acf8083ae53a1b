"""Pins for the oracle's number formats.

Each format is checked against something other than the oracle itself: torch's
own float8_e4m3fn and bfloat16 conversions (library routines), and values that
follow by hand from the format definitions (tests/golden/e4m3_hand_values.txt).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_match_torch():
    ref = _torch_e4m3_values()
    got = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])


def _torch_encode(x):
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448, 448))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_ties_and_random():
    vals = codecs.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2           # exact halfway cases
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    up = np.nextafter(f32(mids), np.float32(1e9))
    dn = np.nextafter(f32(mids), np.float32(-1e9))
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.standard_normal(20000) * 10 ** rng.uniform(-4, 2.7, 20000),
                          rng.uniform(-448, 448, 5000)])
    x = np.concatenate([vals, -vals, mids, -mids, up, dn, -up, rnd]).astype(np.float32)
    got = codecs.e4m3_encode(x.astype(np.float64))
    ref = _torch_encode(x)
    zero = x == 0
    # torch keeps the sign of zero results; the oracle encodes every zero as +0
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    got = np.where((got & 0x7F) == 0, 0, got)
    assert np.array_equal(got[~zero], ref[~zero])


def test_e4m3_saturates_above_448():
    assert codecs.e4m3_encode([1000.0, -1e6, 449.0])[0] == 0x7E
    assert codecs.e4m3_encode([-1e6])[0] == 0xFE


def test_e4m3_hand_values():
    # golden: values derived by hand from the format definition
    path = os.path.join(GOLDEN, "e4m3_hand_values.txt")
    n = 0
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        val, code = line.split()
        v = float.fromhex(val) if val.startswith(("0x", "-0x")) else float(val)
        assert codecs.e4m3_encode([v])[0] == int(code, 16), line
        assert codecs.e4m3_decode([int(code, 16)])[0] == v or abs(v) not in codecs.e4m3_decode(
            np.arange(127, dtype=np.uint8)), line
        n += 1
    assert n >= 10


def test_e2m1_table_closed_form():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert codecs.e2m1_value(c) == mags[c]
        assert codecs.e2m1_value(c | 8) == -mags[c]


def test_e2m1_unpack_order_low_nibble_first():
    # byte 0x21: low nibble 1 (0.5) is element 0, high nibble 2 (1.0) is element 1
    got = codecs.e2m1_unpack(np.array([[0x21, 0xF7]], dtype=np.uint8))
    assert got.tolist() == [[0.5, 1.0, 6.0, -6.0]]


def test_e8m0_closed_form():
    got = codecs.e8m0_decode(np.array([127, 128, 126, 0, 254, 255], dtype=np.uint8))
    assert got[:5].tolist() == [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127]
    assert math.isnan(got[5])


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(50000) * 10 ** rng.uniform(-6, 6, 50000)).astype(np.float32)
    # exact ties: low 16 bits 0x8000, both parities of the kept bit
    bits = rng.integers(0x3F800000, 0x47000000, 2000, dtype=np.uint32)
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_fp32_round_is_ieee_single():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    assert codecs.fp32_round(x).tolist() == [1.0, 1.0 + 2.0 ** -22, float(np.float32(0.1))]
