"""Pins of the plan twin (oracle/plan.py): hand-worked plans and invariants."""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import plan


def _cases():
    with open(os.path.join(GOLDEN, "plan_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_plans(case):
    words = plan.build_plan(**case["args"])
    assert words.tolist() == case["words"]


def check_invariants(words, seqlens, q_len, num_heads, num_cus, topk=0, window=0, topk_lens=None):
    p = plan.unpack(words)
    G, U, S = p["G"], p["U"], p["S"]
    rows = plan.group_rows(seqlens, q_len, topk, window, topk_lens)
    assert G == len(rows)
    assert S <= p["S_max"] == G + U
    assert p["grp_ptr"][0] == 0 and p["grp_ptr"][-1] == S
    assert p["unit_ptr"][0] == 0 and p["unit_ptr"][-1] == S
    assert np.all(np.diff(p["grp_ptr"]) >= 0) and np.all(np.diff(p["unit_ptr"]) >= 0)
    sp = p["splits"]
    # every block of every group covered exactly once, in order
    for g in range(G):
        n = rows[g][1]
        nblk = -(-n // 64)
        mine = sp[p["grp_ptr"][g]:p["grp_ptr"][g + 1]]
        assert np.all(mine[:, 0] == g)
        k = 0
        for s in mine:
            assert s[1] == k and s[2] > s[1]
            k = s[2]
        assert k == nblk
        assert tuple(p["grp_rows"][g]) == rows[g]
    # splits of each unit are where unit_ptr says, and units ascend
    for u in range(U):
        assert np.all(sp[p["unit_ptr"][u]:p["unit_ptr"][u + 1], 3] == u)
    assert np.all(np.diff(sp[:, 3]) >= 0) if S else True
    # cost bound: a unit's blocks plus one overhead per split never exceed quota + FIXED * splits
    for u in range(U):
        mine = sp[p["unit_ptr"][u]:p["unit_ptr"][u + 1]]
        blocks = int((mine[:, 2] - mine[:, 1]).sum()) if len(mine) else 0
        assert blocks <= p["quota"]
    return p


@pytest.mark.parametrize("seed", range(20))
def test_random_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 70))
    Sq = int(rng.integers(1, 5))
    H = int(rng.choice([16, 32, 64, 128]))
    mode = seed % 3
    seqlens = rng.integers(-3, 9000, size=B)
    seqlens[rng.random(B) < 0.1] = 0
    num_cus = int(rng.integers(1, 400))
    if mode == 0:
        w = plan.build_plan(seqlens, Sq, H, num_cus)
        check_invariants(w, seqlens, Sq, H, num_cus)
    elif mode == 1:
        W = int(rng.integers(1, 300))
        w = plan.build_plan(seqlens, Sq, H, num_cus, window=W)
        check_invariants(w, seqlens, Sq, H, num_cus, window=W)
    else:
        topk = int(rng.integers(1, 3000))
        tl = rng.integers(-5, topk + 10, size=B * Sq) if seed % 2 else None
        w = plan.build_plan(seqlens, Sq, H, num_cus, topk=topk, topk_lens=tl)
        check_invariants(w, seqlens, Sq, H, num_cus, topk=topk, topk_lens=tl)


def test_workload_plans():
    from workloads import CONFIGS, make
    for c, spec in CONFIGS.items():
        wl = make(spec) if c != 5 else None
        seqlens = wl.seqlens if wl is not None else np.array(spec.seqlens)
        cus = spec.plan_cus or 256
        w = plan.build_plan(seqlens, spec.q_len, spec.num_heads, cus, spec.topk, spec.window)
        p = check_invariants(w, seqlens, spec.q_len, spec.num_heads, cus, spec.topk, spec.window)
        if c == 1:
            # the tiny workload is planned without splitting
            assert p["S"] == 2 and list(p["grp_ptr"]) == [0, 1, 2]


def test_empty_everything():
    w = plan.build_plan([0, 0, -1], 1, 128, 256)
    p = plan.unpack(w)
    assert p["S"] == 0 and p["total"] == 0 and p["quota"] == 1
    assert list(p["unit_ptr"]) == [0] * (p["U"] + 1)
