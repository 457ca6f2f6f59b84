"""Pins for the oracle's storage decoders (CPU)."""
import math
import os

import numpy as np
import torch

from oracle.formats import decode_bf16, decode_e4m3, e4m3_value_table


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert nan_ours.sum() == 2                      # 0x7F and 0xFF only
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    # signed zeros keep their sign
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_spec_points(golden_dir):
    table = e4m3_value_table()
    n = 0
    with open(os.path.join(golden_dir, "e4m3_spec_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, value = line.split()
            code, value = int(code, 16), float(value)
            if math.isnan(value):
                assert math.isnan(table[code])
            else:
                assert table[code] == value
                assert math.copysign(1.0, table[code]) == math.copysign(1.0, value)
            n += 1
    assert n == 12


def test_e4m3_monotone_and_symmetric():
    t = e4m3_value_table()
    pos = t[:0x7F]                                   # 0x00..0x7E, finite and ordered
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=100000, dtype=np.uint32).astype(np.uint16)
    bits = np.concatenate([bits, np.array([0x0000, 0x8000, 0x3F80, 0x7F80, 0xFF80, 0x0001], np.uint16)])
    ours = decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert decode_bf16(np.array([0x3F80], np.uint16))[0] == 1.0
