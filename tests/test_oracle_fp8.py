"""Pins of the oracle's fp8 decoders (oracle/fp8.py) to things other than themselves."""

import json
import math
import os

import numpy as np
import torch

from conftest import GOLDEN
from oracle import fp8


def _val(v):
    return float("nan") if v == "nan" else float(v)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3fn_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], theirs[~nan])
    # signed zeros kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_printed_values():
    with open(os.path.join(GOLDEN, "ofp8_values.json")) as f:
        g = json.load(f)
    for e in g["e4m3fn"]:
        got = fp8.e4m3fn_value(int(e["code"], 16))
        want = _val(e["value"])
        if math.isnan(want):
            assert math.isnan(got), e
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), e


def test_ue8m0_values():
    with open(os.path.join(GOLDEN, "ofp8_values.json")) as f:
        g = json.load(f)
    for e in g["ue8m0"]:
        got = float(fp8.ue8m0_decode(np.array([int(e["code"], 16)]))[0])
        want = _val(e["value"])
        assert (math.isnan(got) and math.isnan(want)) or got == want, e
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(fp8.ue8m0_decode(codes), ref)
    for k in range(-4, 5):
        assert fp8.ue8m0_decode(np.array([127 + k]))[0] == math.ldexp(1.0, k)


def test_dequant_rows_groups_and_tail():
    rng = np.random.default_rng(0)
    L, d_nope = 5, 448
    codes = rng.integers(0, 256, size=(L, d_nope), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38   # no NaN codes
    scales = np.zeros((L, 8), dtype=np.uint8)
    scales[:, :7] = rng.integers(123, 132, size=(L, 7))
    rope = rng.standard_normal((L, 64))
    out = fp8.dequant_rows(codes, scales, rope)
    assert out.shape == (L, 512)
    for r in range(L):
        for d in (0, 63, 64, 200, 447):
            want = fp8.e4m3fn_value(codes[r, d]) * 2.0 ** (int(scales[r, d // 64]) - 127)
            assert out[r, d] == want
    assert np.array_equal(out[:, 448:], rope)
