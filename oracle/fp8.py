"""fp8 decoding for the latent cache rows — oracle (test infrastructure).

The pages name the formats (HALOps MLA API, mla_attention kv_cache: float8_e4m3fn NoPE values with
one ue8m0 scale per 64 NoPE elements) but do not define them; the definitions used are the OCP
8-bit floating point (OFP8) E4M3 encoding and the OCP Microscaling E8M0 scale encoding:

- e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 is subnormal
  (2^-6 * m/8); no infinities; S.1111.111 is NaN; largest finite 448.
- ue8m0: unsigned 8-bit exponent, value 2^(byte - 127); byte 255 is NaN.

A dequantised NoPE value is e4m3(code) * ue8m0(scale of its 64-wide group), which is exact in
float64 (and in bf16). Pinned by: all 256 codes against torch.float8_e4m3fn, the E8M0 bytes against
torch.float8_e8m0fnu and ldexp, and printed OCP table values (tests/golden/ofp8_values.json).
"""

from __future__ import annotations

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """Elementwise e4m3fn decode of a uint8 array to float64."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def ue8m0_decode(codes: np.ndarray) -> np.ndarray:
    """Elementwise ue8m0 decode: 2^(byte - 127), NaN for 255."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def dequant_rows(nope_codes: np.ndarray, scale_codes: np.ndarray, rope: np.ndarray) -> np.ndarray:
    """Dense float64 rows [L, d_nope + d_rope] from the fp8 row format.

    nope_codes  uint8 [L, d_nope]   e4m3fn NoPE values
    scale_codes uint8 [L, >= ceil(d_nope / 64)]  ue8m0 scale of NoPE group g = columns [64g, 64g+64)
    rope        float [L, d_rope]   the RoPE tail (bf16 values, already widened)
    """
    nope_codes = np.asarray(nope_codes, dtype=np.uint8)
    L, d_nope = nope_codes.shape
    groups = np.arange(d_nope) // 64
    scale = ue8m0_decode(np.asarray(scale_codes)[:, groups]) if L else np.zeros((0, d_nope))
    vals = e4m3fn_decode(nope_codes) * scale
    return np.concatenate([vals, np.asarray(rope, dtype=np.float64)], axis=1)
