"""Pins of the chunked-context plan (oracle/chunks.py)."""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import chunks


def test_golden_plans():
    with open(os.path.join(GOLDEN, "context_chunks_cases.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = chunks.plan_context_chunks(c["lens"], c["W"], c["A"])
        assert [[list(s) for s in ch] for ch in got] == c["chunks"], c["name"]


def test_workspace_smaller_than_alignment_rejected():
    with pytest.raises(ValueError):
        chunks.plan_context_chunks([5], 8, 16)


@pytest.mark.parametrize("W,A", [(64, 1), (64, 16), (100, 16), (4096, 64), (17, 17)])
def test_invariants(W, A):
    rng = np.random.default_rng(W + A)
    for _ in range(200):
        lens = [int(x) for x in rng.integers(0, 3 * W, rng.integers(1, 12))]
        lens = [0 if rng.random() < 0.2 else x for x in lens]
        plan = chunks.plan_context_chunks(lens, W, A)
        # every row covered once, in order
        cursor = {r: 0 for r in range(len(lens))}
        order = []
        for ch in plan:
            assert ch, "no empty chunk"
            assert sum(n for _, _, n in ch) <= W
            reqs = [r for r, _, _ in ch]
            assert reqs == sorted(reqs) and len(set(reqs)) == len(reqs)
            for r, s, n in ch:
                assert n > 0 and s == cursor[r] and s % A == 0
                cursor[r] += n
                order.append(r)
        assert all(cursor[r] == lens[r] for r in range(len(lens)))
        assert order == sorted(order)
        # a chunk closes only when its next aligned piece does not fit (or it is full, or last)
        for ch, nxt in zip(plan, plan[1:]):
            free = W - sum(n for _, _, n in ch)
            r, s, n = nxt[0]
            rem = lens[r] - s
            assert free < A or rem > free or (ch[-1][0] == r and free == 0), (ch, nxt)
            if rem > free:
                assert free // A * A == 0 or (ch[-1][0] == r and ch[-1][1] + ch[-1][2] == s)
