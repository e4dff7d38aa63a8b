"""Sparse MLA prefill over index lists — oracle (test infrastructure).

What is computed (FlashMLA wrapper, flash_mla_sparse_fwd: q, kv, indices, sm_scale, d_v = 512,
returning out, max_logits and lse): each query token t of a prefill attends, with all of its
heads, over the rows of a flat latent buffer kv [s_kv, d_qk] that its own index list names; the
first d_v columns of a row serve as V, as in the absorbed decode. For token t and head h, with J(t)
the entries of indices[t, :] that lie in [0, s_kv) (repeats count once per occurrence):

    s_j         = sm_scale * <q[t, h, :], kv[j, :]>         for j in J(t)
    max_logits  = max_{j in J(t)} s_j                       (-inf when J(t) is empty)
    LSE         = ln sum_{j in J(t)} exp(s_j)               (-inf when J(t) is empty)
    out         = sum_{j in J(t)} exp(s_j - LSE) * kv[j, :d_v]   (0 when J(t) is empty)

Readings where the page leaves a point open (the wrapper gives the signature only):
- q is [s_q, H, d_qk], kv is [s_kv, d_qk] (one latent KV head), indices is [s_q, topk]; entries
  outside [0, s_kv), -1 among them, name no row (the decode's convention for index lists).
- out is [s_q, H, d_v]; lse and max_logits share the LSE layout the wrapper states for the decode,
  (batch, heads, seq_len_q) with one batch: [H, s_q]. Both are in natural-log units of the scaled
  scores, so lse - max_logits lies in [0, ln |J(t)|].

Out, LSE: the decode oracle's attend() on the selected rows (pinned there). max_logits: the
maximum of the same scaled scores. Pinned (tests/test_oracle_sparse_prefill.py) by closed forms (one
visible row: max_logits = LSE = its score and out = its V; equal scores: LSE = max_logits + ln n and
out = the mean of the V rows), by pure-Python brute force on tiny inputs, by the bound
0 <= LSE - max_logits <= ln |J|, and by the decode oracle on the same rows.
"""

from __future__ import annotations

import numpy as np

from .attention import attend, visible_sparse


def sparse_prefill(q: np.ndarray, kv: np.ndarray, indices: np.ndarray, sm_scale: float,
                   d_v: int = 512, tokens=None, abs_mass: bool = False):
    """Returns out [n, H, d_v], max_logits [H, n], lse [H, n] in float64 for the tokens listed in
    `tokens` (all s_q tokens when None, n = s_q); with abs_mass also A [n, H, d_v] = sum_j P_j |V_j|
    (see attention.attend)."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    idx = np.asarray(indices, dtype=np.int64)
    s_q, H, _ = q.shape
    s_kv = kv.shape[0]
    toks = list(range(s_q)) if tokens is None else [int(t) for t in tokens]
    n = len(toks)
    out = np.zeros((n, H, d_v))
    mlog = np.full((H, n), -np.inf)
    lse = np.zeros((H, n))
    A = np.zeros((n, H, d_v)) if abs_mass else None
    for i, t in enumerate(toks):
        J = visible_sparse(s_kv, idx[t])
        rows = kv[J]
        if J.size > 0:
            mlog[:, i] = (sm_scale * (q[t] @ rows.T)).max(axis=1)
        res = attend(q[t], rows, sm_scale, d_v, None, abs_mass)
        out[i] = res[0]
        lse[:, i] = res[1]
        if abs_mass:
            A[i] = res[2]
    return (out, mlog, lse, A) if abs_mass else (out, mlog, lse)
