"""Gathering context rows from the paged cache into a dense workspace — oracle (test infrastructure).

vLLM mla_attention.py, _compute_prefill_context: gather_and_maybe_dequant_cache(src_cache, dst,
block_table, cu_seq_lens, token_to_seq, num_tokens, ..., seq_starts) puts the context rows of one
chunk of requests into a contiguous workspace for the up-projection: output row i belongs to request
r = token_to_seq[i] and holds its logical row seq_starts[r] + i - cu_seq_lens[r], dequantised when
the cache holds fp8 rows.

Reading: rows whose position or page falls outside the block table or the cache are zeros (the
GPU writes zeros instead of reading outside the cache).

Pinned (tests/test_oracle_gather.py) against the depager of oracle/paging.py on whole requests and
on request spans.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .fp8 import dequant_rows
from .paging import _bf16_bytes_to_f64


def gather_context(cache: np.ndarray, block_table: np.ndarray, cu_seq_lens: np.ndarray,
                   seq_starts: Optional[np.ndarray], token_to_seq: np.ndarray, kv_format: str,
                   d_qk: int, d_rope: int, page_size: int) -> np.ndarray:
    """float64 [n, d_qk] gathered rows."""
    cache = np.asarray(cache, dtype=np.uint8)
    num_pages = cache.shape[0]
    bt = np.asarray(block_table)
    n = len(token_to_seq)
    d_nope = d_qk - d_rope
    row_bytes = 2 * d_qk if kv_format == "bf16" else d_nope + 2 * d_rope
    out = np.zeros((n, d_qk))
    for i in range(n):
        r = int(token_to_seq[i])
        j = (0 if seq_starts is None else int(seq_starts[r])) + i - int(cu_seq_lens[r])
        if j < 0 or j // page_size >= bt.shape[1]:
            continue
        page = int(bt[r, j // page_size])
        if page < 0 or page >= num_pages:
            continue
        slot = j % page_size
        raw = cache[page, slot * row_bytes:(slot + 1) * row_bytes]
        if kv_format == "bf16":
            out[i] = _bf16_bytes_to_f64(raw)
        else:
            s = page_size * row_bytes + 8 * slot
            scales = cache[page, s:s + 8][None, :]
            rope = _bf16_bytes_to_f64(raw[d_nope:])[None, :]
            out[i] = dequant_rows(raw[None, :d_nope], scales, rope)[0]
    return out
