"""Log-sum-exp merge of attention partials — oracle (test infrastructure).

Split-KV partials are combined by their log-sum-exps (vLLM merge_attn_states in the chunked-prefill
description of mla_attention.py; HALOps mla_output_proj, "split-KV LSE combine"):

    LSE = ln sum_i exp(LSE_i),     O = sum_i exp(LSE_i - LSE) * O_i

where partial i covers a disjoint subset of the visible rows, O_i is normalised by its own softmax
denominator and LSE_i is its log-sum-exp. A partial with no rows is (O_i = 0, LSE_i = -inf) and
carries no weight (vLLM neutralize_empty_context_partials). Partials never include the sink; the
sink is folded in once after the merge (HALOps attn_sink: one extra denominator term):

    LSE' = ln(exp(LSE) + exp(sink)),   O' = O * exp(LSE - LSE')

Pinned by: merged == unsplit attention over random split points including empty splits, in float64
(tests/test_oracle_attention.py).
"""

from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from .attention import attend


def merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]], d_v: Optional[int] = None):
    """Merge partials [(O_i [M, d_v], LSE_i [M])] into (O [M, d_v], LSE [M])."""
    if len(parts) == 0:
        raise ValueError("merge needs at least one partial (use an empty partial for none)")
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])     # [n, M]
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])     # [n, M, d_v]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe[None, :]), 0.0)    # [n, M]
    s = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, s, 1.0)), -np.inf)
    coef = np.where(finite[None, :], w / np.where(finite, s, 1.0)[None, :], 0.0)
    O = np.einsum("nm,nmd->md", coef, outs)
    return O, lse


def fold_sink(O: np.ndarray, lse: np.ndarray, sink: np.ndarray):
    """Add exp(sink) to each row's denominator after a merge."""
    lse = np.asarray(lse, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    new = np.logaddexp(lse, sink)
    scale = np.where(np.isfinite(lse), np.exp(lse - new), 0.0)
    return np.asarray(O, dtype=np.float64) * scale[:, None], new


def split_partials(q_rows: np.ndarray, K: np.ndarray, sm_scale: float, d_v: int,
                   bounds: Sequence[int]) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Partials of attention over the row ranges [bounds[i], bounds[i+1]) (no sink)."""
    return [attend(q_rows, K[bounds[i]:bounds[i + 1]], sm_scale, d_v)
            for i in range(len(bounds) - 1)]
