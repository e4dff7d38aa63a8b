"""The host chunk planner of the C ABI (mla_plan_context_chunks) against the chunk-plan oracle:
identical plans (integer work, bit-exact). Runs on the CPU: the planner is host code."""

import ctypes

import numpy as np
import pytest

import mla_paged_latent_plan_amd as mla
from mla_paged_latent_plan_amd import _lib
from oracle import chunks


@pytest.mark.parametrize("W,A", [(64, 1), (64, 16), (100, 16), (4096, 64), (16, 16), (65536, 64)])
def test_planner_matches_oracle(W, A):
    rng = np.random.default_rng(W * 7 + A)
    for _ in range(150):
        n = int(rng.integers(0, 14))
        lens = rng.integers(0, 3 * W, n)
        lens[rng.random(n) < 0.2] = 0
        assert mla.plan_context_chunks(lens, W, A) == chunks.plan_context_chunks(lens.tolist(), W, A)


def test_planner_rejects_and_reports_capacity():
    lib = _lib.load()
    lens = np.array([100, 50], dtype=np.int32)
    out = [np.zeros(16, dtype=np.int32) for _ in range(5)]
    args = lambda W, A, mc, ms: (2, lens.ctypes.data, W, A, mc, ms, out[0].ctypes.data,
                                 out[1].ctypes.data, out[2].ctypes.data, out[3].ctypes.data,
                                 out[4].ctypes.data)
    assert lib.mla_plan_context_chunks(*args(8, 16, 8, 8)) == 2      # W < alignment
    assert lib.mla_plan_context_chunks(*args(64, 16, 1, 8)) == 6     # more chunks than room
    assert lib.mla_plan_context_chunks(*args(64, 16, 8, 1)) == 6     # more spans than room
    assert lib.mla_plan_context_chunks(*args(64, 16, 8, 8)) == 0
    assert out[0][0] == 3  # 100 = 64 + 36; 36 + 16 (aligned share of 50) = 52; 34 left
