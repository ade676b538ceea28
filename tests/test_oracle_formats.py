"""Pins of the oracle's number-format decoders.

The fp8 format is the one the serving flags name (``--kv-cache-dtype fp8_e4m3``
in the SGLang post's launch example), read as OCP E4M3FN.  Each decoder is
checked against torch's own casts (a library routine independent of the
oracle) over every code, and against spot values that follow from the format
definitions.
"""
import math

import numpy as np
import torch


def test_e4m3_all_codes_match_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_mod.e4m3_values(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert nan_ours.sum() == 2                      # 0x7F and 0xFF only, no infinities
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])


def test_e4m3_spot_values(oracle_mod):
    v = lambda c: float(oracle_mod.e4m3_values(np.array([c], np.uint8))[0])  # noqa: E731
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x38) == 1.0                           # exponent field 7 = bias
    assert v(0x7E) == 448.0                         # largest finite
    assert v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6                     # smallest normal
    assert v(0x01) == 2.0 ** -9                     # smallest subnormal: 2^-6 * 1/8
    assert v(0x07) == 7 * 2.0 ** -9                 # largest subnormal
    assert v(0x3C) == 1.5                           # 1 + 4/8
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))


def test_bf16_all_codes_match_torch(oracle_mod):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.bf16_values(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all()
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])


def test_bf16_spot_values(oracle_mod):
    v = lambda c: float(oracle_mod.bf16_values(np.array([c], np.uint16))[0])  # noqa: E731
    assert v(0x3F80) == 1.0
    assert v(0xC000) == -2.0
    assert v(0x0001) == 2.0 ** -133                 # smallest subnormal
    assert v(0x7F80) == math.inf and v(0xFF80) == -math.inf
    assert v(0x3FC0) == 1.5
