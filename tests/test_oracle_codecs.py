"""Pins for the oracle's storage-format decoders (CPU only).

The E4M3FN decoder is checked against torch's float8_e4m3fn cast over all 256
codes and against values the OCP format definition fixes; the BF16 decoder
against torch's bfloat16.  Neither check re-runs the oracle's own formula.
"""
import math

import numpy as np
import pytest
import torch

from oracle.codecs import e4m3_decode, bf16_decode


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # sign of zero too
    assert math.copysign(1.0, ours[0x80]) == -1.0


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0xB8, -1.0), (0x30, 0.5), (0x77, 240.0), (0x78, 256.0),
])
def test_e4m3_format_values(code, value):
    assert e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3_nan_codes_only():
    v = e4m3_decode(np.arange(256, dtype=np.uint8))
    assert set(np.flatnonzero(np.isnan(v)).tolist()) == {0x7F, 0xFF}


def test_e4m3_positive_codes_increase():
    v = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000).astype(np.uint16)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = bf16_decode(bits)
    nan = np.isnan(ref_t)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref_t[~nan])


@pytest.mark.parametrize("bits,value", [(0x3F80, 1.0), (0xC000, -2.0), (0x0000, 0.0),
                                        (0x7F80, math.inf), (0x3F00, 0.5)])
def test_bf16_format_values(bits, value):
    assert bf16_decode(np.array([bits], dtype=np.uint16))[0] == value
