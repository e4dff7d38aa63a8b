"""Expanded (MHA-form) MLA attention — oracle (test infrastructure), used only as a pin.

vLLM mla_attention.py module docstring, "Compute Friendly Approach": per head n the keys and values
are up-projected from the latent rows,

    k_nope = kv_c @ W_UK[:, n, :]      (Skv x P)
    v      = kv_c @ W_UV[:, n, :]      (Skv x V)
    score  = sm_scale * (q_nope[s, n] . k_nope[j] + q_pe[s, n] . k_pe[j])

and each head runs ordinary softmax attention with QK head dim P + R and V head dim V. The
"Data-Movement Friendly Approach" of the same docstring folds W_UK into the query and W_UV into the
output, which is the form the decode path computes; the two must agree, which pins attention.py.
This module deliberately writes its own softmax rather than calling attention.py.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def expanded_attention(q_nope: np.ndarray, q_pe: np.ndarray, kv_c: np.ndarray, k_pe: np.ndarray,
                       W_UK: np.ndarray, W_UV: np.ndarray, sm_scale: float,
                       visible: list, sink: Optional[np.ndarray] = None):
    """q_nope [Sq, N, P], q_pe [Sq, N, R], kv_c [Skv, Lkv], k_pe [Skv, R], W_UK [Lkv, N, P],
    W_UV [Lkv, N, V]; visible[s] = row positions visible to query s.
    Returns (o [Sq, N, V], lse [N, Sq])."""
    Sq, N, P = q_nope.shape
    V = W_UV.shape[2]
    o = np.zeros((Sq, N, V))
    lse = np.zeros((N, Sq))
    for n in range(N):
        k_nope = kv_c @ W_UK[:, n, :]            # [Skv, P]
        v = kv_c @ W_UV[:, n, :]                 # [Skv, V]
        for s in range(Sq):
            J = np.asarray(visible[s], dtype=np.int64)
            sc = sm_scale * (k_nope[J] @ q_nope[s, n] + k_pe[J] @ q_pe[s, n])
            if sink is not None:
                sc_all = np.concatenate([sc, [sink[n]]])
            else:
                sc_all = sc
            if sc_all.size == 0:
                lse[n, s] = -np.inf
                continue
            mx = sc_all.max()
            z = np.exp(sc_all - mx).sum()
            lse[n, s] = mx + np.log(z)
            w = np.exp(sc - lse[n, s])
            o[s, n] = w @ v[J]
    return o, lse
