"""Pins of the sparse prefill oracle (oracle/sparse_prefill.py)."""

import math

import numpy as np

from oracle import attention, brute
from oracle.sparse_prefill import sparse_prefill


def _case(rng, s_q=5, H=3, d_qk=24, d_v=16, s_kv=11, topk=7):
    q = rng.standard_normal((s_q, H, d_qk))
    kv = rng.standard_normal((s_kv, d_qk))
    idx = rng.integers(-2, s_kv + 3, size=(s_q, topk))
    return q, kv, idx


def test_brute_force_tiny():
    rng = np.random.default_rng(7)
    q, kv, idx = _case(rng)
    scale = 0.31
    out, mlog, lse = sparse_prefill(q, kv, idx, scale, d_v=16)
    for t in range(q.shape[0]):
        vis = [int(j) for j in idx[t] if 0 <= j < kv.shape[0]]
        O_b, L_b = brute.decode_token(q[t].tolist(), kv.tolist(), vis, scale, 16)
        np.testing.assert_allclose(out[t], np.array(O_b), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[:, t], np.array(L_b), rtol=1e-12, atol=1e-12)
        for h in range(q.shape[1]):
            best = -math.inf
            for j in vis:
                best = max(best, scale * sum(a * b for a, b in zip(q[t, h], kv[j])))
            assert mlog[h, t] == best or abs(mlog[h, t] - best) <= 1e-12 * max(1.0, abs(best))


def test_single_visible_row_closed_form():
    rng = np.random.default_rng(1)
    q, kv, _ = _case(rng, s_q=2, topk=4)
    idx = np.array([[3, -1, 11, 40], [-5, 0, 99, 11]])  # one valid entry per token
    scale = 0.5
    out, mlog, lse = sparse_prefill(q, kv, idx, scale, d_v=16)
    for t, j in ((0, 3), (1, 0)):
        s = scale * q[t] @ kv[j]
        np.testing.assert_allclose(mlog[:, t], s, rtol=1e-13)
        np.testing.assert_allclose(lse[:, t], s, rtol=1e-13)
        np.testing.assert_allclose(out[t], np.broadcast_to(kv[j, :16], (q.shape[1], 16)), rtol=1e-13)


def test_equal_scores_closed_form():
    """q = 0: every visible score is 0, so max_logits = 0, LSE = ln n, out = mean of V rows."""
    rng = np.random.default_rng(2)
    _, kv, _ = _case(rng)
    q = np.zeros((2, 3, 24))
    idx = np.array([[1, 4, 4, 9, -1, 30, 2], [5, 5, 5, 5, 5, 5, 5]])
    out, mlog, lse = sparse_prefill(q, kv, idx, 1.0, d_v=16)
    np.testing.assert_array_equal(mlog, 0.0)
    np.testing.assert_allclose(lse[:, 0], math.log(5), rtol=1e-14)
    np.testing.assert_allclose(lse[:, 1], math.log(7), rtol=1e-14)
    mean0 = kv[[1, 4, 4, 9, 2], :16].mean(axis=0)
    np.testing.assert_allclose(out[0], np.broadcast_to(mean0, (3, 16)), rtol=1e-13)
    np.testing.assert_allclose(out[1], np.broadcast_to(kv[5, :16], (3, 16)), rtol=1e-13)


def test_empty_rows():
    rng = np.random.default_rng(3)
    q, kv, _ = _case(rng, s_q=1)
    idx = np.array([[-1, -1, 11, 12, -7, 100, 11]])
    out, mlog, lse = sparse_prefill(q, kv, idx, 0.2, d_v=16)
    assert np.all(out == 0) and np.all(np.isneginf(mlog)) and np.all(np.isneginf(lse))


def test_lse_bounds_and_decode_oracle():
    """0 <= LSE - max <= ln |J|, and out / LSE equal the decode oracle's with one request."""
    rng = np.random.default_rng(4)
    q, kv, idx = _case(rng, s_q=6, topk=9)
    scale = 0.7
    out, mlog, lse = sparse_prefill(q, kv, idx, scale, d_v=16)
    for t in range(6):
        n = int(((idx[t] >= 0) & (idx[t] < kv.shape[0])).sum())
        if n == 0:
            continue
        gap = lse[:, t] - mlog[:, t]
        assert np.all(gap >= -1e-12) and np.all(gap <= math.log(n) + 1e-12)
    O_d, L_d = attention.mla_decode(q[None], lambda b: kv, [kv.shape[0]], scale, d_v=16,
                                    indices=idx[None])
    np.testing.assert_allclose(out, O_d[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, L_d[0], rtol=1e-13, atol=1e-13)


def test_token_subset():
    rng = np.random.default_rng(5)
    q, kv, idx = _case(rng, s_q=6)
    full = sparse_prefill(q, kv, idx, 0.4, d_v=16)
    part = sparse_prefill(q, kv, idx, 0.4, d_v=16, tokens=[4, 1])
    np.testing.assert_array_equal(part[0], full[0][[4, 1]])
    np.testing.assert_array_equal(part[1], full[1][:, [4, 1]])
    np.testing.assert_array_equal(part[2], full[2][:, [4, 1]])


def test_planted_mistake_negative_index_wraps():
    """Reading -1 as Python's last row would let kv[-1] (the best-scoring row here) into the max."""
    kv = np.zeros((4, 24))
    kv[3, 0] = 10.0
    kv[1, 0] = 1.0
    q = np.zeros((1, 1, 24))
    q[0, 0, 0] = 1.0
    idx = np.array([[1, -1]])
    _, mlog, _ = sparse_prefill(q, kv, idx, 1.0, d_v=16)
    assert mlog[0, 0] == 1.0
    planted = (q[0] @ kv[idx[0]].T).max()  # what unchecked indexing gives
    assert planted == 10.0 != mlog[0, 0]
