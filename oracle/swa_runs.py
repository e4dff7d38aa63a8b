"""Run-compressed sliding-window plan — oracle (test infrastructure), integer arithmetic only.

HALOps MLA API, mla_attention_plan. A token's SWA window is given as the cache slots s_0, s_1, ...
of its rows (kv_indices [T, topk], the first topk_lengths[t] columns valid). Rows g - 1 and g are
in one run iff s_g == s_{g-1} + kv_run_step (1 or -1) and s_g // page_size == s_{g-1} // page_size.
A window with at most two runs is described by them; one with more (a padding or not yet written
window) is described by its row 0 alone. The result per token is (slot0, len0, slot1, rows): rows is
the effective length, the first len0 rows form the first run.

Readings where the page leaves a point open:
- Row g of a run starting at slot s sits at s + kv_run_step * g (the page writes slot0 + g, which
  is the kv_run_step = 1 case; with -1 consecutive rows descend).
- rows = clamp(topk_lengths[t], 0, topk), or topk when no lengths are given.
- One run: slot1 = -1 (a second run exists exactly when len0 < rows; it may itself start at a
  padding slot -1). Empty window: (-1, 0, -1, 0). A cut window: (kv[t, 0], 1, -1, 1).
- page(slot) = floor(slot / page_size), so a negative (padding) slot inside the length breaks a
  run like any other slot.

Pinned (tests/test_oracle_swa_runs.py) by hand-worked windows and by brute force: the runs
reproduce every slot of an uncut window, the first run is maximal, and windows with three or more
runs are exactly the cut ones.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def page_of(slot: int, page_size: int) -> int:
    return slot // page_size  # floor division, also for negative slots


def window_runs(slots: Sequence[int], n: int, page_size: int, step: int):
    """(slot0, len0, slot1, rows) of one window whose first n entries are valid."""
    if n <= 0:
        return (-1, 0, -1, 0)
    # indices g (1 <= g < n) where a new run starts
    starts = [g for g in range(1, n)
              if slots[g] != slots[g - 1] + step or page_of(slots[g], page_size) != page_of(slots[g - 1], page_size)]
    if len(starts) == 0:
        return (int(slots[0]), n, -1, n)
    if len(starts) == 1:
        return (int(slots[0]), starts[0], int(slots[starts[0]]), n)
    return (int(slots[0]), 1, -1, 1)


def swa_runs(kv_indices: np.ndarray, topk_lengths: Optional[np.ndarray], page_size: int,
             step: int) -> np.ndarray:
    """int32 [T, 4] plan rows (slot0, len0, slot1, rows) for every token."""
    kv = np.asarray(kv_indices, dtype=np.int64)
    T, topk = kv.shape
    out = np.zeros((T, 4), dtype=np.int32)
    for t in range(T):
        n = topk if topk_lengths is None else min(max(int(topk_lengths[t]), 0), topk)
        out[t] = window_runs(kv[t].tolist(), n, page_size, step)
    return out
