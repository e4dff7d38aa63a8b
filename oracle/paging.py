"""Reading a paged latent cache back into dense rows — oracle (test infrastructure).

The block table maps a request's logical page i to a physical page (FlashMLA wrapper: k_cache
(num_blocks, page_size, num_heads_k, head_dim) with block_table (batch, max_blocks) int32; MLA has
one KV head). Logical row j of request b lives on physical page block_table[b, j // page_size] at
slot j % page_size. Row formats:

- bf16: a page is page_size rows of d_qk bfloat16 values.
- fp8 (HALOps mla_attention, kv_cache): a page is page_size rows of [d_nope e4m3fn bytes]
  [d_rope bfloat16], followed by page_size 8-byte slots holding the row's ue8m0 scales, one per 64
  NoPE values.

Written independently of the input generator; pinned by round trips through it under different
page permutations (tests/test_workloads.py).
"""

from __future__ import annotations

import numpy as np

from .fp8 import dequant_rows


def _bf16_bytes_to_f64(b: np.ndarray) -> np.ndarray:
    """Little-endian bf16 byte pairs [..., 2k] -> float64 [..., k]: bf16 is the top half of fp32."""
    u16 = np.ascontiguousarray(b).view("<u2").astype(np.uint32)
    return (u16 << 16).view("<f4").astype(np.float64)


def logical_row_bytes(cache: np.ndarray, block_table: np.ndarray, b: int, L: int, page_size: int,
                      row_bytes: int) -> np.ndarray:
    """Raw bytes [L, row_bytes] of the first L logical rows of request b."""
    cache = np.asarray(cache)
    j = np.arange(L)
    page = np.asarray(block_table)[b, j // page_size].astype(np.int64)
    slot = j % page_size
    out = np.empty((L, row_bytes), dtype=np.uint8)
    for r in range(L):
        s = int(slot[r]) * row_bytes
        out[r] = cache[page[r], s:s + row_bytes]
    return out


def dense_rows(cache: np.ndarray, block_table: np.ndarray, b: int, L: int, kv_format: str,
               d_qk: int, d_rope: int, page_size: int) -> np.ndarray:
    """Dense float64 rows [L, d_qk] of request b, decoded from the paged cache."""
    if kv_format == "bf16":
        raw = logical_row_bytes(cache, block_table, b, L, page_size, 2 * d_qk)
        return _bf16_bytes_to_f64(raw)
    d_nope = d_qk - d_rope
    row_bytes = d_nope + 2 * d_rope
    raw = logical_row_bytes(cache, block_table, b, L, page_size, row_bytes)
    cache = np.asarray(cache)
    j = np.arange(L)
    page = np.asarray(block_table)[b, j // page_size].astype(np.int64)
    slot = j % page_size
    base = page_size * row_bytes
    scales = np.empty((L, 8), dtype=np.uint8)
    for r in range(L):
        s = base + int(slot[r]) * 8
        scales[r] = cache[page[r], s:s + 8]
    rope = _bf16_bytes_to_f64(raw[:, d_nope:])
    return dequant_rows(raw[:, :d_nope], scales, rope)
