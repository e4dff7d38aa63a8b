"""Writing new tokens' latent rows into the paged cache — oracle (test infrastructure).

What is computed (vLLM mla_attention.py, `update_kv_cache(kv_c_normed, k_pe, kv_cache,
slot_mapping, ...)`; HALOps MLA API, mla_attention `kv_cache`: each token's new row is written in
place): token i's row [kv_c_i, k_pe_i] lands in cache slot slot_mapping[i], i.e. physical page
slot // page_size, row slot % page_size of that page.

- bf16 rows: the d_qk bfloat16 values are stored as they are.
- fp8 rows (HALOps kv_cache layout: [d_nope e4m3fn][d_rope bfloat16] per row, then one 8-byte
  ue8m0 scale slot per row after the page's rows): each 64-wide group of kv_c gets one ue8m0
  scale byte and 64 e4m3fn codes; k_pe is stored as bfloat16; the pad bytes of the scale slot
  (one for d_nope = 448) are zero.

The pages do not say how the scale of a group is chosen. Reading used here (and by the HIP
kernel): with amax the largest |value| of the group, the scale is 2^k for the smallest integer k
such that amax <= 448 * 2^k (448 = largest finite e4m3fn), k clamped to [-127, 127]; the byte is
127 + k. An all-zero group gets byte 127 (scale 1). Each code is the e4m3fn value nearest to
value * 2^-k, ties to the even code (round to nearest even); |value * 2^-k| <= 448 by the choice of
k, so no code saturates. Slots that are negative or beyond the cache are skipped (vLLM marks
tokens without a slot with -1); repeated slots are outside the contract.

Pinned by (tests/test_oracle_kvwrite.py): the encoder against torch's float8_e4m3fn cast on
random values and on every midpoint between neighbouring codes, decode-then-encode identity on
all 254 finite codes, the closed-form scale bytes at and next to the powers of two, the relative
error bound 2^-4 of round-to-nearest with 3 mantissa bits, and the written bytes read back through
the decoder of oracle/fp8.py and the depager of oracle/paging.py.
"""

from __future__ import annotations

import math

import numpy as np

from .fp8 import e4m3fn_value

E4M3_MAX = 448.0

# finite non-negative e4m3fn magnitudes in code order (codes 0x00 .. 0x7E): increasing
_MAGS = np.array([e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)


def e4m3fn_encode(y: float) -> int:
    """e4m3fn code of y, rounded to the nearest representable value, ties to the even code.

    Requires |y| <= 448 (the scale rule guarantees it). The sign of zero is kept (-0.0 -> 0x80)."""
    y = float(y)
    if not (abs(y) <= E4M3_MAX):
        raise ValueError(f"{y} is outside the finite e4m3fn range")
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0x00
    a = abs(y)
    hi = int(np.searchsorted(_MAGS, a, side="left"))  # first magnitude >= a
    if hi < len(_MAGS) and _MAGS[hi] == a:
        return sign | hi
    lo = hi - 1  # _MAGS[lo] < a < _MAGS[hi]
    dl, dh = a - _MAGS[lo], _MAGS[hi] - a
    if dl < dh:
        code = lo
    elif dh < dl:
        code = hi
    else:
        code = lo if lo % 2 == 0 else hi  # the even code: mantissa bit 0 clear
    return sign | code


def scale_exponent(amax: float) -> int:
    """k of the group scale 2^k: smallest integer with amax <= 448 * 2^k, clamped to [-127, 127];
    0 for an all-zero group."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    k = math.ceil(math.log2(amax / E4M3_MAX))
    # guard the float log against being one off at exact powers of two
    while amax > E4M3_MAX * 2.0 ** k:
        k += 1
    while amax <= E4M3_MAX * 2.0 ** (k - 1):
        k -= 1
    return max(-127, min(127, k))


def quantize_group(x: np.ndarray):
    """(scale byte, e4m3fn codes) of one group of values (float64, exact bf16 values)."""
    x = np.asarray(x, dtype=np.float64)
    k = scale_exponent(np.max(np.abs(x)) if x.size else 0.0)
    codes = np.array([e4m3fn_encode(math.ldexp(v, -k)) for v in x], dtype=np.uint8)
    return 127 + k, codes


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of values that are exactly representable in bfloat16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(v, dtype=np.float64), equal_nan=True):
        raise ValueError("values are not exact bfloat16")
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not exact bfloat16")
    return (u >> 16).astype(np.uint16)


def encode_row(kv_c: np.ndarray, k_pe: np.ndarray, kv_format: str) -> tuple:
    """Bytes of one cache row and (fp8 only) its 8-byte scale slot.

    kv_c  float64 [d_nope] (bf16 values), k_pe float64 [d_rope] (bf16 values)."""
    kv_c = np.asarray(kv_c, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    if kv_format == "bf16":
        row = np.concatenate([bf16_bits(kv_c), bf16_bits(k_pe)]).view(np.uint8)
        return row, None
    if kv_format != "fp8":
        raise ValueError(kv_format)
    d_nope = kv_c.shape[0]
    if d_nope % 64 != 0 or d_nope // 64 > 8:
        raise ValueError("d_nope must be a multiple of 64, at most 512")
    codes = np.zeros(d_nope, dtype=np.uint8)
    slot = np.zeros(8, dtype=np.uint8)
    for g in range(d_nope // 64):
        sb, c = quantize_group(kv_c[64 * g:64 * g + 64])
        slot[g] = sb
        codes[64 * g:64 * g + 64] = c
    row = np.concatenate([codes, bf16_bits(k_pe).view(np.uint8)])
    return row, slot


def write_rows(cache: np.ndarray, kv_format: str, page_size: int, kv_c: np.ndarray,
               k_pe: np.ndarray, slot_mapping: np.ndarray) -> np.ndarray:
    """Copy of cache (uint8 [num_pages, page_stride]) with token i's row written at slot_mapping[i].

    kv_c float64 [n, d_nope], k_pe float64 [n, d_rope] (bf16 values); slot_mapping int [n]."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    num_pages = out.shape[0]
    n, d_nope = kv_c.shape
    d_rope = k_pe.shape[1]
    row_bytes = 2 * (d_nope + d_rope) if kv_format == "bf16" else d_nope + 2 * d_rope
    for i in range(n):
        s = int(slot_mapping[i])
        if s < 0 or s // page_size >= num_pages:
            continue
        page, r = divmod(s, page_size)
        row, slot = encode_row(kv_c[i], k_pe[i], kv_format)
        out[page, r * row_bytes:(r + 1) * row_bytes] = row
        if slot is not None:
            off = page_size * row_bytes + 8 * r
            out[page, off:off + 8] = slot
    return out
