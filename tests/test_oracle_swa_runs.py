"""Pins of the run-compressed window plan (oracle/swa_runs.py)."""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import swa_runs


def test_golden_windows():
    with open(os.path.join(GOLDEN, "swa_runs_cases.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = swa_runs.window_runs(c["slots"], c["n"], c["page_size"], c["step"])
        assert list(got) == c["runs"], (c["name"], got)


def _slots_of(runs, step):
    slot0, len0, slot1, rows = runs
    return [slot0 + step * g if g < len0 else slot1 + step * (g - len0) for g in range(rows)]


def _random_window(rng, page_size, step, W):
    """A window of W rows in a ring of slots, possibly wrapping, crossing pages or padded."""
    kind = rng.integers(0, 5)
    base = int(rng.integers(0, 40 * page_size))
    slots = [base + step * g for g in range(W)]
    if kind == 1:    # ring wrap: the tail continues from another place
        cut = int(rng.integers(1, W))
        other = int(rng.integers(0, 40 * page_size))
        slots = slots[:cut] + [other + step * g for g in range(W - cut)]
    elif kind == 2:  # padding inside the window
        for g in rng.choice(W, size=min(W, int(rng.integers(1, 4))), replace=False):
            slots[g] = -1
    elif kind == 3:  # a not yet written window: scattered slots
        slots = [int(x) for x in rng.integers(-1, 40 * page_size, W)]
    return slots


@pytest.mark.parametrize("page_size,step", [(64, 1), (64, -1), (16, 1), (1, 1)])
def test_runs_reproduce_uncut_windows(page_size, step):
    rng = np.random.default_rng(page_size + step)
    for _ in range(300):
        W = int(rng.integers(1, 140))
        slots = _random_window(rng, page_size, step, W)
        n = int(rng.integers(0, W + 1))
        runs = swa_runs.window_runs(slots, n, page_size, step)
        # brute force: count the runs of the first n slots by walking them
        nruns = 0
        for g in range(n):
            if g == 0 or slots[g] != slots[g - 1] + step or (slots[g] // page_size) != (slots[g - 1] // page_size):
                nruns += 1
        if n == 0:
            assert runs == (-1, 0, -1, 0)
        elif nruns <= 2:
            assert runs[3] == n and _slots_of(runs, step) == slots[:n]
            # the first run is maximal and every run stays on one page
            assert runs[1] == n or slots[runs[1]] != slots[runs[1] - 1] + step or \
                (slots[runs[1]] // page_size) != (slots[runs[1] - 1] // page_size)
            rows = _slots_of(runs, step)
            for g in range(1, runs[1]):
                assert rows[g] // page_size == rows[0] // page_size
            assert (runs[1] == runs[3]) == (nruns == 1)  # a second run exactly when len0 < rows
        else:
            assert runs == (slots[0], 1, -1, 1)


def test_lengths_clamped_and_defaulted():
    kv = np.array([[5, 6, 7, 8], [9, 10, 30, 31]], dtype=np.int32)
    np.testing.assert_array_equal(swa_runs.swa_runs(kv, None, 64, 1), [[5, 4, -1, 4], [9, 2, 30, 4]])
    np.testing.assert_array_equal(swa_runs.swa_runs(kv, np.array([9, -2]), 64, 1),
                                  [[5, 4, -1, 4], [-1, 0, -1, 0]])


def test_planted_mistake_page_boundary_ignored():
    """A run that ignores page boundaries would merge slots 63 and 64 (pages 0 and 1)."""
    slots = [62, 63, 64, 65]
    good = swa_runs.window_runs(slots, 4, 64, 1)
    assert good == (62, 2, 64, 4)
    planted = (62, 4, -1, 4)  # what a step-only rule gives
    assert planted != good
