"""Weight absorption around the decode — oracle (test infrastructure).

vLLM mla_attention.py (forward_mqa and _v_up_proj; module docstring, "Data-Movement Friendly
Approach"): the query's NoPE part is multiplied into the latent space per head before the decode,
ql_nope[b, n, :] = q_nope[b, n, :] x W_UK_T[n] (W_UK_T: (N, P, L)), and the decode's latent output
is multiplied back per head after it, out[b, n, :] = o[b, n, :] x W_UV[n] (W_UV: (N, L, V)). The
decode's query is [ql_nope, q_pe] (q_pe is already rotated).

Weight layouts used here are the per-head packed ones the pages' CPU (AMX) path keeps, with the
contraction index contiguous: w_uk [N, L, P] (w_uk[n, l, p] = W_UK[l, n, p] of the (L, N, P)
weight the pages dequantise from kv_b_proj) and w_uv [N, V, L] (w_uv[n, v, l] = W_UV[l, n, v]).

Pinned (tests/test_oracle_absorb.py) by the absorbed form agreeing with the expanded MHA form of
oracle/mha.py, which up-projects the rows instead and never calls these functions.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def q_absorb(q_nope: np.ndarray, w_uk: np.ndarray, q_pe: Optional[np.ndarray] = None) -> np.ndarray:
    """Decode query [T, N, L (+ R)] from q_nope [T, N, P], w_uk [N, L, P] and q_pe [T, N, R]."""
    T, N, P = q_nope.shape
    ql = np.empty((T, N, w_uk.shape[1]))
    for n in range(N):
        ql[:, n, :] = np.asarray(q_nope[:, n, :], dtype=np.float64) @ np.asarray(w_uk[n], dtype=np.float64).T
    if q_pe is None:
        return ql
    return np.concatenate([ql, np.asarray(q_pe, dtype=np.float64)], axis=2)


def v_up(o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Per-head output [T, N, V] from the latent output o [T, N, L] and w_uv [N, V, L]."""
    T, N, L = o.shape
    out = np.empty((T, N, w_uv.shape[1]))
    for n in range(N):
        out[:, n, :] = np.asarray(o[:, n, :], dtype=np.float64) @ np.asarray(w_uv[n], dtype=np.float64).T
    return out
