"""Absorbed-form MLA decode attention on dense rows — oracle (test infrastructure).

What is computed (vLLM mla_attention.py module docstring, "Data-Movement Friendly Approach"): every
head's query [ql_nope, q_pe] (d_qk wide) attends over rows K = [kv_c, k_pe] shared by all heads,
and the latent part kv_c (the first d_v columns of each row) also serves as V. For request b, query
token t and head h:

    s_j  = sm_scale * <q[b,t,h,:], K_b[j,:]>                 for j in the visible set J(b,t)
    LSE  = ln( sum_{j in J} exp(s_j) + exp(sink_h) )          (sink term only if a sink is given)
    O    = sum_{j in J} exp(s_j - LSE) * K_b[j, :d_v]

Visible sets:
- positions (vLLM MLACommonMetadata comment on context_len / query_len / seq_len): the Sq new
  tokens are the last Sq positions of a sequence of length L, so token t sits at pos_t = L - Sq + t;
- causal: j <= pos_t (multi-token verify at consecutive positions, HALOps mla_attention);
- window W: j >= pos_t - W + 1, the window including the token's own row (HALOps
  mla_attention_plan, topk_lengths);
- sparse: the entries k < topk_len of the index list indices[b,t,:] with 0 <= idx < L, counted per
  occurrence (FlashMLA wrapper, indices (batch, seq_len_q, topk); HALOps: entries past a token's
  length are ignored).

The sink (HALOps mla_attention, attn_sink) is a per-head logit in the same domain as the scaled
scores, added once to the softmax denominator; the returned LSE includes it. An empty visible set
gives O = 0 and LSE = -inf (or LSE = sink_h), the empty-partial convention of vLLM
neutralize_empty_context_partials.

Output layouts follow the FlashMLA wrapper's I/O contract: O [B, Sq, H, d_v], LSE [B, H, Sq].
All arithmetic is float64 with a max-subtracted log-sum-exp; numpy's matmul is the only library
primitive. Pinned by: brute force (brute.py), closed forms, the expanded MHA form (mha.py),
split-and-merge (merge.py) and fp64 torch.logsumexp / torch.softmax (tests/test_oracle_attention.py).
"""

from __future__ import annotations

from typing import Callable, Optional, Tuple

import numpy as np


def visible_dense(L: int, Sq: int, t: int, causal: bool, window: int) -> np.ndarray:
    """Sorted positions j visible to query token t of a dense (non-index) request of length L."""
    L = max(int(L), 0)
    pos = L - Sq + t
    lo, hi = 0, L - 1
    if causal:
        hi = min(hi, pos)
    if window > 0:
        lo = max(lo, pos - window + 1)
    if hi < lo:
        return np.zeros(0, dtype=np.int64)
    return np.arange(lo, hi + 1, dtype=np.int64)


def visible_sparse(L: int, idx_row: np.ndarray, n: Optional[int] = None) -> np.ndarray:
    """Positions listed by an index row: the first n entries that lie in [0, L), with repeats."""
    idx = np.asarray(idx_row, dtype=np.int64)
    if n is not None:
        idx = idx[:max(int(n), 0)]
    return idx[(idx >= 0) & (idx < max(int(L), 0))]


def attend(q_rows: np.ndarray, K: np.ndarray, sm_scale: float, d_v: int,
           sink: Optional[np.ndarray] = None, abs_mass: bool = False):
    """Softmax attention of query rows [M, d_qk] over rows K [n, d_qk]; V = K[:, :d_v].

    sink: optional [M] logits added to each row's denominator. Returns (O [M, d_v], LSE [M]);
    with abs_mass also A [M, d_v] = sum_j P_j |V_j|, the weighted magnitude of the terms that
    make up O (the scale of any error proportional to the probabilities, e.g. their rounding).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    M = q_rows.shape[0]
    n = K.shape[0]
    if n == 0:
        O = np.zeros((M, d_v))
        lse = np.full(M, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64).copy()
        return (O, lse, np.zeros((M, d_v))) if abs_mass else (O, lse)
    S = sm_scale * (q_rows @ K.T)                      # [M, n]
    m = S.max(axis=1)
    if sink is not None:
        m = np.maximum(m, np.asarray(sink, dtype=np.float64))
    E = np.exp(S - m[:, None])
    denom = E.sum(axis=1)
    if sink is not None:
        denom = denom + np.exp(np.asarray(sink, dtype=np.float64) - m)
    lse = m + np.log(denom)
    P = np.exp(S - lse[:, None])
    O = P @ K[:, :d_v]
    if abs_mass:
        return O, lse, P @ np.abs(K[:, :d_v])
    return O, lse


def mla_decode(q: np.ndarray, rows_of: Callable[[int], np.ndarray], seqlens, sm_scale: float,
               d_v: int = 512, causal: bool = False, window: int = 0,
               indices: Optional[np.ndarray] = None, topk_lens: Optional[np.ndarray] = None,
               sink: Optional[np.ndarray] = None, abs_mass: bool = False):
    """Reference decode over all requests.

    q        [B, Sq, H, d_qk] (any float dtype; widened to float64)
    rows_of  b -> dense float64 rows K_b [L_b, d_qk] of request b (logical order)
    seqlens  [B] sequence lengths L_b (including the Sq new tokens)
    indices  optional [B, Sq, topk] request-local positions (sparse mode)
    topk_lens optional [B * Sq] number of leading index entries used per token
    sink     optional [H] per-head sink logits
    Returns O [B, Sq, H, d_v] and LSE [B, H, Sq], float64; with abs_mass also A [B, Sq, H, d_v]
    (see attend).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Sq, H, _ = q.shape
    O = np.zeros((B, Sq, H, d_v))
    LSE = np.zeros((B, H, Sq))
    A = np.zeros((B, Sq, H, d_v)) if abs_mass else None
    sink_v = None if sink is None else np.asarray(sink, dtype=np.float64)
    for b in range(B):
        L = int(seqlens[b])
        K = rows_of(b) if L > 0 else np.zeros((0, q.shape[3]))
        for t in range(Sq):
            if indices is not None:
                n = None if topk_lens is None else int(topk_lens[b * Sq + t])
                J = visible_sparse(L, np.asarray(indices)[b, t], n)
            else:
                J = visible_dense(L, Sq, t, causal, window)
            res = attend(q[b, t], K[J], sm_scale, d_v, sink_v, abs_mass)
            O[b, t] = res[0]
            LSE[b, :, t] = res[1]
            if abs_mass:
                A[b, t] = res[2]
    return (O, LSE, A) if abs_mass else (O, LSE)
