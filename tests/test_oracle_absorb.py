"""Pins of the absorption oracle (oracle/absorb.py): absorbed == expanded MHA (oracle/mha.py)."""

import math

import numpy as np
import pytest

from oracle import absorb, attention, mha


@pytest.mark.parametrize("Sq,causal", [(1, False), (3, True)])
def test_absorb_then_decode_then_up_equals_expanded(Sq, causal):
    rng = np.random.default_rng(40 + Sq)
    N, P, R, Lkv, V, Skv = 4, 16, 8, 32, 12, 9
    W_UK = rng.standard_normal((Lkv, N, P)) / 4     # the pages' (L, N, P) weight
    W_UV = rng.standard_normal((Lkv, N, V)) / 4     # the pages' (L, N, V) weight
    kv_c = rng.standard_normal((Skv, Lkv))
    k_pe = rng.standard_normal((Skv, R))
    q_nope = rng.standard_normal((Sq, N, P))
    q_pe = rng.standard_normal((Sq, N, R))
    scale = 1 / math.sqrt(P + R)
    vis = [attention.visible_dense(Skv, Sq, t, causal, 0).tolist() for t in range(Sq)]
    o_mha, lse_mha = mha.expanded_attention(q_nope, q_pe, kv_c, k_pe, W_UK, W_UV, scale, vis)
    w_uk = np.transpose(W_UK, (1, 0, 2))            # [N, L, P]
    w_uv = np.transpose(W_UV, (1, 2, 0))            # [N, V, L]
    q_lat = absorb.q_absorb(q_nope, w_uk, q_pe)     # [Sq, N, L + R]
    assert q_lat.shape == (Sq, N, Lkv + R)
    rows = np.concatenate([kv_c, k_pe], axis=1)
    O_lat, lse_lat = attention.mla_decode(q_lat[None], lambda b: rows, [Skv], scale, Lkv, causal, 0)
    o_abs = absorb.v_up(O_lat[0], w_uv)
    np.testing.assert_allclose(o_abs, o_mha, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse_lat[0], lse_mha, rtol=1e-12)


def test_planted_transpose_is_caught():
    """Using w_uk[n] untransposed (a plausible layout mistake) breaks the identity."""
    rng = np.random.default_rng(3)
    N, P, L = 2, 8, 8
    q = rng.standard_normal((3, N, P))
    w = rng.standard_normal((N, L, P))
    good = absorb.q_absorb(q, w)
    bad = np.stack([q[:, n, :] @ w[n] for n in range(N)], axis=1)
    assert not np.allclose(good, bad)
