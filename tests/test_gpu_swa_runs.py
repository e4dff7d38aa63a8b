"""GPU parity of mla_swa_runs (through the C ABI) against the run-compressed window oracle:
bit-exact integer plan rows."""

import numpy as np
import pytest
import torch

from oracle import swa_runs

pytestmark = pytest.mark.gpu


def _windows(T, topk, page_size, step, seed):
    """Seeded windows of a ring of slots: plain runs, wraps, page crossings, padding, scattered."""
    rng = np.random.default_rng(seed)
    kv = np.full((T, topk), -1, dtype=np.int32)
    lengths = rng.integers(-2, topk + 3, T).astype(np.int32)
    for t in range(T):
        kind = rng.integers(0, 6)
        base = int(rng.integers(0, 50 * page_size))
        row = [base + step * g for g in range(topk)]
        if kind == 1:
            cut = int(rng.integers(1, topk)) if topk > 1 else 0
            other = int(rng.integers(0, 50 * page_size))
            row = row[:cut] + [other + step * g for g in range(topk - cut)]
        elif kind == 2:
            for g in rng.choice(topk, size=min(topk, 3), replace=False):
                row[g] = -1
        elif kind == 3:
            row = [int(x) for x in rng.integers(-1, 50 * page_size, topk)]
        elif kind == 4:  # a window that starts just before a page boundary
            b = (int(rng.integers(1, 50)) * page_size) - int(rng.integers(0, 4)) * step
            row = [b + step * g for g in range(topk)]
        kv[t] = np.maximum(np.array(row, dtype=np.int64), -1).astype(np.int32)
    return kv, lengths


@pytest.mark.parametrize("T,topk,page_size,step,use_len", [
    (640, 131, 64, 1, True), (640, 131, 64, -1, True), (333, 64, 16, 1, False),
    (100, 200, 1, 1, True), (7, 1, 64, 1, True), (128, 128, 64, 1, False)])
def test_swa_runs_bit_exact(T, topk, page_size, step, use_len):
    import mla_paged_latent_plan_amd as mla
    kv, lengths = _windows(T, topk, page_size, step, seed=T + topk + page_size)
    runs = torch.full((T, 4), 12345, dtype=torch.int32, device="cuda")
    print(f"[gpu] swa_runs T={T} topk={topk} page={page_size} step={step}", flush=True)
    mla.mla_swa_runs(torch.from_numpy(kv).cuda(), torch.from_numpy(lengths).cuda() if use_len else None,
                     page_size, step, runs)
    torch.cuda.synchronize()
    want = swa_runs.swa_runs(kv, lengths if use_len else None, page_size, step)
    got = runs.cpu().numpy()
    bad = np.argwhere(np.any(got != want, axis=1))
    assert bad.size == 0, f"{len(bad)} tokens differ, first {bad[:3].ravel().tolist()}: " \
                          f"{got[bad[0][0]].tolist()} vs {want[bad[0][0]].tolist()}"
