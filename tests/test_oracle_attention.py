"""Pins of the attention oracle (oracle/attention.py, merge.py) to brute force, closed forms, the
expanded MHA form, library routines and hand-derived values."""

import json
import math
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import attention, brute, merge, mha


def _f(v):
    return -math.inf if v == "-inf" else float(v)


def _golden():
    with open(os.path.join(GOLDEN, "tiny_attention.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_golden_attend(case):
    d = len(case["q"][0])
    rows = np.asarray(case["rows"], dtype=np.float64).reshape(-1, d)
    sink = None if case["sink"] is None else np.asarray(case["sink"])
    O, lse = attention.attend(np.asarray(case["q"]), rows, case["sm_scale"], case["d_v"], sink)
    np.testing.assert_allclose(O, np.asarray(case["O"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.asarray(case["lse"]), rtol=0, atol=1e-14)


def test_golden_merge():
    c = _golden()["merge_cases"][0]
    parts = [(np.asarray(p["O"]), np.asarray([_f(x) for x in p["lse"]])) for p in c["parts"]]
    O, lse = merge.merge(parts)
    np.testing.assert_allclose(O, np.asarray(c["O"]), atol=1e-14)
    np.testing.assert_allclose(lse, np.asarray(c["lse"]), atol=1e-14)


@pytest.mark.parametrize("case", _golden()["position_cases"], ids=str)
def test_golden_positions(case):
    for t, want in enumerate(case["visible"]):
        got = attention.visible_dense(case["L"], case["Sq"], t, case["causal"], case["window"])
        assert got.tolist() == want


def _rand_case(rng, L, Sq, H, d, topk=0):
    q = rng.standard_normal((1, Sq, H, d))
    K = rng.standard_normal((L, d))
    idx = None
    if topk:
        idx = rng.integers(-2, L + 2, size=(1, Sq, topk))
    return q, K, idx


@pytest.mark.parametrize("mode", ["dense", "causal", "window", "sparse", "sink", "sink_window"])
@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_brute_force_tiny(mode, L):
    rng = np.random.default_rng(100 + L)
    Sq = 1 if mode in ("dense", "sink") else min(3, L + 1)
    H, d, dv = 3, 6, 4
    q, K, idx = _rand_case(rng, L, Sq, H, d, topk=5 if mode == "sparse" else 0)
    causal = mode in ("causal", "window", "sink_window")
    window = 2 if "window" in mode else 0
    sink = rng.standard_normal(H) if "sink" in mode else None
    O, lse = attention.mla_decode(q, lambda b: K, [L], 0.37, dv, causal, window, idx, None, sink)
    for t in range(Sq):
        if idx is not None:
            vis = [int(j) for j in idx[0, t] if 0 <= j < L]
        else:
            pos = L - Sq + t
            vis = [j for j in range(L) if (not causal or j <= pos) and (window == 0 or j >= pos - window + 1)]
        bo, bl = brute.decode_token(q[0, t].tolist(), K.tolist(), vis, 0.37, dv,
                                    None if sink is None else sink.tolist())
        np.testing.assert_allclose(O[0, t], np.asarray(bo), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[0, :, t], np.asarray(bl), rtol=1e-12, atol=1e-12)


def test_closed_form_single_row():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 9))
    K = rng.standard_normal((1, 9))
    O, lse = attention.attend(q, K, 0.5, 7)
    np.testing.assert_array_equal(O, np.broadcast_to(K[0, :7], (4, 7)))
    np.testing.assert_allclose(lse, 0.5 * q @ K[0], rtol=1e-15)
    sink = rng.standard_normal(4)
    O, lse = attention.attend(q, K, 0.5, 7, sink)
    s0 = 0.5 * q @ K[0]
    sig = 1.0 / (1.0 + np.exp(sink - s0))
    np.testing.assert_allclose(O, sig[:, None] * K[0, :7][None, :], rtol=1e-13)
    np.testing.assert_allclose(lse, np.logaddexp(s0, sink), rtol=1e-14)


def test_closed_form_uniform_scores():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((37, 10))
    O, lse = attention.attend(np.zeros((3, 10)), K, 1.0, 6)
    np.testing.assert_allclose(O, np.broadcast_to(K[:, :6].mean(axis=0), (3, 6)), rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(37.0), rtol=1e-15)
    sink = np.array([0.0, 1.0, -2.0])
    O, lse = attention.attend(np.zeros((3, 10)), K, 1.0, 6, sink)
    np.testing.assert_allclose(lse, np.log(37.0 + np.exp(sink)), rtol=1e-14)
    np.testing.assert_allclose(O, (37.0 / (37.0 + np.exp(sink)))[:, None] * K[:, :6].mean(axis=0), rtol=1e-13)


def test_closed_form_identical_rows():
    rng = np.random.default_rng(3)
    row = rng.standard_normal(12)
    K = np.tile(row, (20, 1))
    O, _ = attention.attend(rng.standard_normal((5, 12)) * 3, K, 0.8, 10)
    np.testing.assert_allclose(O, np.broadcast_to(row[:10], (5, 10)), rtol=1e-13)


def test_library_logsumexp_softmax():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((16, 576))
    K = rng.standard_normal((300, 576))
    O, lse = attention.attend(q, K, 1 / math.sqrt(192), 512)
    S = torch.from_numpy(q) @ torch.from_numpy(K).T / math.sqrt(192)
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=1).numpy(), rtol=1e-13)
    P = torch.softmax(S, dim=1)
    np.testing.assert_allclose(O, (P @ torch.from_numpy(K[:, :512])).numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_split_merge_equals_unsplit(seed):
    rng = np.random.default_rng(10 + seed)
    n = int(rng.integers(1, 200))
    q = rng.standard_normal((8, 64)) * 2
    K = rng.standard_normal((n, 64))
    cuts = sorted(rng.integers(0, n + 1, size=int(rng.integers(1, 6))).tolist())
    bounds = [0] + cuts + [n]                 # repeats give empty splits
    parts = merge.split_partials(q, K, 0.3, 32, bounds)
    O, lse = merge.merge(parts)
    O0, lse0 = attention.attend(q, K, 0.3, 32)
    np.testing.assert_allclose(O, O0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse0, rtol=1e-13)
    sink = rng.standard_normal(8)
    Os, lses = merge.fold_sink(O, lse, sink)
    O1, lse1 = attention.attend(q, K, 0.3, 32, sink)
    np.testing.assert_allclose(Os, O1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lses, lse1, rtol=1e-13)


def test_merge_all_empty():
    e = (np.zeros((2, 4)), np.full(2, -np.inf))
    O, lse = merge.merge([e, e])
    assert np.all(O == 0) and np.all(np.isneginf(lse))
    O, lse = merge.fold_sink(O, lse, np.array([0.5, -1.0]))
    assert np.all(O == 0)
    np.testing.assert_array_equal(lse, [0.5, -1.0])


@pytest.mark.parametrize("Sq,causal,window", [(1, False, 0), (3, True, 0), (3, True, 2), (2, False, 0)])
def test_absorbed_equals_expanded(Sq, causal, window):
    rng = np.random.default_rng(20 + Sq)
    N, P, R, Lkv, V, Skv = 4, 16, 8, 32, 16, 9
    W_UK = rng.standard_normal((Lkv, N, P)) / 4
    W_UV = rng.standard_normal((Lkv, N, V)) / 4
    kv_c = rng.standard_normal((Skv, Lkv))
    k_pe = rng.standard_normal((Skv, R))
    q_nope = rng.standard_normal((Sq, N, P))
    q_pe = rng.standard_normal((Sq, N, R))
    sink = rng.standard_normal(N)
    scale = 1 / math.sqrt(P + R)
    vis = [attention.visible_dense(Skv, Sq, t, causal, window).tolist() for t in range(Sq)]
    o_mha, lse_mha = mha.expanded_attention(q_nope, q_pe, kv_c, k_pe, W_UK, W_UV, scale, vis, sink)
    # absorbed: ql_nope[s,n,l] = sum_p q_nope[s,n,p] W_UK[l,n,p]; query [ql_nope, q_pe]; rows [kv_c, k_pe]
    ql_nope = np.einsum("snp,lnp->snl", q_nope, W_UK)
    q_lat = np.concatenate([ql_nope, q_pe], axis=2)[None]
    rows = np.concatenate([kv_c, k_pe], axis=1)
    O_lat, lse_lat = attention.mla_decode(q_lat, lambda b: rows, [Skv], scale, Lkv, causal, window,
                                          sink=sink)
    o_abs = np.einsum("snl,lnv->snv", O_lat[0], W_UV)
    np.testing.assert_allclose(o_abs, o_mha, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse_lat[0], lse_mha, rtol=1e-12)


def test_verify_equals_decode():
    """Token t of a causal Sq-token verify equals a one-token decode of the first L - Sq + 1 + t rows."""
    rng = np.random.default_rng(30)
    L, Sq, H, d = 23, 4, 5, 40
    q = rng.standard_normal((1, Sq, H, d))
    K = rng.standard_normal((L, d))
    for window in (0, 6):
        O, lse = attention.mla_decode(q, lambda b: K, [L], 0.2, 32, True, window)
        for t in range(Sq):
            Lt = L - Sq + 1 + t
            O1, lse1 = attention.mla_decode(q[:, t:t + 1], lambda b: K[:Lt], [Lt], 0.2, 32, False, window)
            np.testing.assert_array_equal(O[0, t], O1[0, 0])
            np.testing.assert_array_equal(lse[0, :, t], lse1[0, :, 0])


def test_sparse_equals_dense():
    rng = np.random.default_rng(31)
    L, H, d = 50, 4, 24
    q = rng.standard_normal((1, 1, H, d))
    K = rng.standard_normal((L, d))
    Od, lsed = attention.mla_decode(q, lambda b: K, [L], 0.3, 16)
    idx = rng.permutation(L)[None, None, :]
    Os, lses = attention.mla_decode(q, lambda b: K, [L], 0.3, 16, indices=idx)
    np.testing.assert_allclose(Os, Od, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lses, lsed, rtol=1e-13)
    # a window expressed as an index list equals the native window
    Sq, W = 3, 7
    q3 = rng.standard_normal((1, Sq, H, d))
    Ow, lsew = attention.mla_decode(q3, lambda b: K, [L], 0.3, 16, True, W)
    idx = np.full((1, Sq, W + 3), -1)
    for t in range(Sq):
        pos = L - Sq + t
        idx[0, t, :W] = np.arange(pos - W + 1, pos + 1)[::-1]
    Oi, lsei = attention.mla_decode(q3, lambda b: K, [L], 0.3, 16, indices=idx)
    np.testing.assert_allclose(Oi, Ow, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lsei, lsew, rtol=1e-13)


def test_topk_lens_and_invalid_indices():
    rng = np.random.default_rng(32)
    L, H, d = 20, 2, 8
    q = rng.standard_normal((1, 2, H, d))
    K = rng.standard_normal((L, d))
    idx = np.array([[[3, -1, 25, 7, 7, 1], [2, 4, 6, 8, 10, 12]]])
    O, lse = attention.mla_decode(q, lambda b: K, [L], 1.0, 8, indices=idx, topk_lens=[5, 0])
    bo, bl = brute.decode_token(q[0, 0].tolist(), K.tolist(), [3, 7, 7], 1.0, 8)
    np.testing.assert_allclose(O[0, 0], bo, rtol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], bl, rtol=1e-12)
    assert np.all(O[0, 1] == 0) and np.all(np.isneginf(lse[0, :, 1]))


def test_row_order_invariance():
    rng = np.random.default_rng(33)
    q = rng.standard_normal((6, 30))
    K = rng.standard_normal((45, 30))
    O, lse = attention.attend(q, K, 0.4, 20)
    p = rng.permutation(45)
    O2, lse2 = attention.attend(q, K[p], 0.4, 20)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_planted_mistakes_are_caught(monkeypatch):
    """Plausible slips in the oracle's attend (dropped scale, sink left out of the returned LSE, V
    taken from the wrong end of the row) must fail the brute-force pin."""
    rng = np.random.default_rng(40)
    q = rng.standard_normal((1, 1, 3, 6))
    K = rng.standard_normal((4, 6))
    sink = rng.standard_normal(3)
    bo, bl = brute.decode_token(q[0, 0].tolist(), K.tolist(), [0, 1, 2, 3], 0.37, 4, sink.tolist())
    good = attention.attend

    def no_scale(qr, KK, s, dv, sk=None, am=False):
        return good(qr, KK, 1.0, dv, sk)

    def sink_dropped_from_lse(qr, KK, s, dv, sk=None, am=False):
        O, _ = good(qr, KK, s, dv, sk)
        _, lse = good(qr, KK, s, dv, None)
        return O, lse

    def v_from_tail(qr, KK, s, dv, sk=None, am=False):
        O, lse = good(qr, KK, s, dv, sk)
        P = np.exp(s * (qr @ KK.T) - lse[:, None])
        return P @ KK[:, -dv:], lse

    for bad in (no_scale, sink_dropped_from_lse, v_from_tail):
        monkeypatch.setattr(attention, "attend", bad)
        O, lse = attention.mla_decode(q, lambda b: K, [4], 0.37, 4, sink=sink)
        caught = not (np.allclose(O[0, 0], bo, atol=1e-9) and np.allclose(lse[0, :, 0], bl, atol=1e-9))
        assert caught, bad.__name__
    monkeypatch.setattr(attention, "attend", good)


def test_abs_mass_closed_forms():
    """The weighted magnitude sum_j P_j |V_j|: equals |O| when every V entry of a column has one
    sign, and equals the plain mean of |V| for uniform scores."""
    rng = np.random.default_rng(41)
    K = np.abs(rng.standard_normal((7, 8)))
    q = rng.standard_normal((3, 8))
    O, _, A = attention.attend(q, K, 0.3, 5, abs_mass=True)
    np.testing.assert_allclose(A, np.abs(O), rtol=1e-12)
    K2 = rng.standard_normal((7, 8))
    O2, lse2, A2 = attention.attend(np.zeros((2, 8)), K2, 0.3, 5, abs_mass=True)
    np.testing.assert_allclose(A2, np.broadcast_to(np.abs(K2[:, :5]).mean(axis=0), (2, 5)), rtol=1e-12)
    np.testing.assert_allclose(lse2, np.log(7.0), rtol=1e-12)
