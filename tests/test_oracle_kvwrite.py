"""Pins of the cache-write oracle (oracle/kvwrite.py) to things other than itself."""

import math

import numpy as np
import pytest
import torch

from oracle import fp8, kvwrite, paging

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_encode_inverts_decode_on_every_finite_code():
    for c in FINITE:
        assert kvwrite.e4m3fn_encode(fp8.e4m3fn_value(c)) == c, hex(c)


def test_encoder_matches_torch_cast_on_random_values():
    # torch's float8_e4m3fn cast rounds to nearest even; below 448 it never saturates
    g = np.random.default_rng(7)
    y = np.concatenate([g.uniform(-448, 448, 4000), g.normal(0, 1, 4000),
                        g.normal(0, 1, 4000) * 2.0 ** -8, [0.0, -0.0, 448.0, -448.0]])
    y = y.astype(np.float32).astype(np.float64)  # values an fp32 kernel would hold exactly
    ours = np.array([kvwrite.e4m3fn_encode(v) for v in y], dtype=np.uint8)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_encoder_ties_go_to_even_codes():
    # every midpoint between neighbouring finite magnitudes: nearest-even picks the even code,
    # and torch's cast agrees
    mags = [fp8.e4m3fn_value(c) for c in range(0x7F)]
    mids = np.array([(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])])
    for i, m in enumerate(mids):
        want = i if i % 2 == 0 else i + 1
        assert kvwrite.e4m3fn_encode(m) == want
        assert kvwrite.e4m3fn_encode(-m) == 0x80 | want
    theirs = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([kvwrite.e4m3fn_encode(m) for m in mids], dtype=np.uint8)
    assert np.array_equal(ours, theirs)


def test_encoder_rejects_values_past_448():
    with pytest.raises(ValueError):
        kvwrite.e4m3fn_encode(449.0)


@pytest.mark.parametrize("k", [-127, -20, -1, 0, 1, 5, 100])
def test_scale_exponent_closed_forms(k):
    top = 448.0 * 2.0 ** k
    assert kvwrite.scale_exponent(top) == k              # exactly 448 * 2^k fits 2^k
    if k < 127:
        assert kvwrite.scale_exponent(top * (1 + 2 ** -20)) == k + 1
    if k > -127:
        assert kvwrite.scale_exponent(top / 2) == k - 1  # 224 * 2^k fits 2^(k-1)


def test_scale_exponent_zero_and_clamps():
    assert kvwrite.scale_exponent(0.0) == 0
    assert kvwrite.scale_exponent(2.0 ** -140) == -127
    assert kvwrite.scale_exponent(1.0) == -8   # 1 <= 448 / 256 = 1.75, 1 > 448 / 512


def test_quantized_group_error_bound():
    # round to nearest with 3 mantissa bits: relative error <= 2^-4 for values that land in the
    # normal e4m3 range, absolute error <= 2^-10 * scale below it
    g = np.random.default_rng(3)
    for t in range(50):
        x = g.normal(0, 1, 64) * 2.0 ** g.integers(-30, 30)
        x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
        sb, codes = kvwrite.quantize_group(x)
        scale = 2.0 ** (sb - 127)
        back = fp8.e4m3fn_decode(codes) * scale
        assert np.max(np.abs(back)) <= 448 * scale
        assert np.max(np.abs(x)) <= 448 * scale and (np.max(np.abs(x)) > 224 * scale)
        normal = np.abs(x) >= 2.0 ** -6 * scale
        assert np.all(np.abs(back - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
        assert np.all(np.abs(back - x)[~normal] <= 2.0 ** -10 * scale)


def test_all_zero_group():
    sb, codes = kvwrite.quantize_group(np.array([0.0] * 63 + [-0.0]))
    assert sb == 127
    assert np.all(codes[:63] == 0) and codes[63] == 0x80


def test_exactly_representable_groups_round_trip():
    # values e4m3(c) * 2^k whose group holds a full-range code come back exactly
    g = np.random.default_rng(11)
    for k in (-9, 0, 4):
        c = g.choice(FINITE, 64)
        c[5] = 0x7E  # 448: the group's amax is 448 * 2^k, so the scale is exactly 2^k
        x = fp8.e4m3fn_decode(c) * 2.0 ** k
        sb, codes = kvwrite.quantize_group(x)
        assert sb == 127 + k
        assert np.array_equal(fp8.e4m3fn_decode(codes), fp8.e4m3fn_decode(c))


@pytest.mark.parametrize("fmt,d_qk", [("bf16", 576), ("fp8", 576), ("fp8", 512)])
def test_written_rows_read_back(fmt, d_qk):
    """Rows written at slots are found by the depager through a block table: bf16 rows exactly,
    fp8 rows as their quantised values (pad byte of the scale slot zero)."""
    d_rope, page_size, num_pages = 64, 16, 5
    d_nope = d_qk - d_rope
    row_bytes = 2 * d_qk if fmt == "bf16" else d_nope + 2 * d_rope
    stride = page_size * row_bytes + (8 * page_size if fmt == "fp8" else 0)
    cache = np.full((num_pages, stride), 0xFF, dtype=np.uint8)
    g = torch.Generator().manual_seed(5)
    L = 40
    kv_c = (torch.randn(L, d_nope, generator=g) * 3).to(torch.bfloat16).to(torch.float64).numpy()
    k_pe = torch.randn(L, d_rope, generator=g).to(torch.bfloat16).to(torch.float64).numpy()
    bt = np.array([[3, 0, 4]], dtype=np.int32)  # logical pages 0, 1, 2 of one request
    slots = np.array([bt[0, j // page_size] * page_size + j % page_size for j in range(L)])
    slots_skip = slots.copy()
    slots_skip[7] = -1                      # skipped
    out = kvwrite.write_rows(cache, fmt, page_size, kv_c, k_pe, slots_skip)
    # a slot past the cache is skipped too
    out2 = kvwrite.write_rows(out, fmt, page_size, kv_c[:1], k_pe[:1],
                              np.array([num_pages * page_size]))
    assert np.array_equal(out, out2)
    rows = paging.dense_rows(out, bt, 0, L, fmt, d_qk, d_rope, page_size)
    want_pe = k_pe
    if fmt == "bf16":
        want_c = kv_c
    else:
        want_c = np.empty_like(kv_c)
        for i in range(L):
            for gi in range(d_nope // 64):
                sb, codes = kvwrite.quantize_group(kv_c[i, 64 * gi:64 * gi + 64])
                want_c[i, 64 * gi:64 * gi + 64] = fp8.e4m3fn_decode(codes) * 2.0 ** (sb - 127)
    keep = np.arange(L) != 7
    assert np.array_equal(rows[keep, :d_nope], want_c[keep])
    assert np.array_equal(rows[keep, d_nope:], want_pe[keep])
    assert np.all(np.isnan(rows[7]))        # the skipped row keeps its old (poison) bytes
    if fmt == "fp8" and d_nope == 448:
        r = 3
        off = page_size * row_bytes + 8 * r
        assert out[bt[0, 0], off + 7] == 0


def test_planted_mistakes_are_caught():
    """Truncation instead of rounding, or a scale one power too large, fails the pins above."""
    y = np.array([1.12, 3.4, 0.0107], dtype=np.float64)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    trunc = []
    for v in y:  # largest magnitude not above v
        hi = int(np.searchsorted(kvwrite._MAGS, abs(v), side="right")) - 1
        trunc.append(hi)
    assert not np.array_equal(np.array(trunc, dtype=np.uint8), theirs)
    # a scale rule of floor(log2(amax / 448)) + 1 gives 448 * 2^k the scale 2^(k+1), which the
    # closed form (exactly 2^k) rejects
    planted = math.floor(math.log2(448.0 * 4 / 448.0)) + 1
    assert planted != 2 and kvwrite.scale_exponent(448.0 * 4) == 2
