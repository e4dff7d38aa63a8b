"""The input generator's paged cache read back by the oracle's own depager."""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import fp8, paging
from workloads import CONFIGS, Spec, cache_layout, make


def _logical_dense(wl, b):
    s = wl.spec
    r = wl.request_rows(b)
    if s.kv_format == "bf16":
        return r.to(torch.float64).numpy()
    nope, scales, rope = r
    return fp8.dequant_rows(nope.numpy(), scales.numpy(), rope.to(torch.float64).numpy())


SMALL = [
    Spec("t_bf16", batch=3, q_len=1, num_heads=16, page_size=16, seqlens=(1, 40, 77), seed=5),
    Spec("t_fp8_576", batch=3, q_len=1, num_heads=16, kv_format="fp8", page_size=16,
         seqlens=(33, 0, 64), seed=6),
    Spec("t_fp8_512", batch=2, q_len=4, num_heads=8, d_qk=512, kv_format="fp8", page_size=64,
         seqlens=(130, 5), seed=7),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_depager_round_trip(spec):
    wl = make(spec)
    for b in range(spec.batch):
        L = int(wl.seqlens[b])
        got = paging.dense_rows(wl.cache.numpy(), wl.block_table.numpy(), b, L, spec.kv_format,
                                spec.d_qk, spec.d_rope, spec.page_size)
        want = _logical_dense(wl, b)
        assert got.shape == want.shape
        assert np.array_equal(got, want)


def test_page_permutation_changes_pages_not_rows():
    spec = SMALL[1]
    a = make(dataclasses.replace(spec, page_seed=1))
    b = make(dataclasses.replace(spec, page_seed=2))
    assert not np.array_equal(a.block_table.numpy(), b.block_table.numpy())
    assert not np.array_equal(a.cache.numpy(), b.cache.numpy())
    for r in range(spec.batch):
        L = int(a.seqlens[r])
        ra = paging.dense_rows(a.cache.numpy(), a.block_table.numpy(), r, L, "fp8", 576, 64, 16)
        rb = paging.dense_rows(b.cache.numpy(), b.block_table.numpy(), r, L, "fp8", 576, 64, 16)
        assert np.array_equal(ra, rb, equal_nan=False)


def test_layout_sizes():
    assert cache_layout("bf16", 576, 64, 64)["page_stride"] == 64 * 1152
    l3 = cache_layout("fp8", 576, 64, 64)
    assert l3["row_bytes"] == 640 and l3["page_stride"] == 41600
    l4 = cache_layout("fp8", 512, 64, 64)
    assert l4["row_bytes"] == 576 and l4["page_stride"] == 37440   # HALOps: a multiple of 576


def test_poison_outside_rows():
    spec = SMALL[1]
    wl = make(spec)
    lay = cache_layout("fp8", 576, 64, 16)
    used = set()
    bt = wl.block_table.numpy()
    for b in range(spec.batch):
        n = -(-int(wl.seqlens[b]) // 16)
        used.update(bt[b, :n].tolist())
    unused = [p for p in range(wl.num_pages) if p not in used]
    assert unused and np.all(wl.cache.numpy()[unused] == 0xFF)
    # tail slot of request 0's only page (33 rows -> 3 pages, last holds 1 row)
    last = bt[0, 2]
    assert np.all(wl.cache.numpy()[last, lay["row_bytes"]:16 * lay["row_bytes"]] == 0xFF)


def test_configs_shapes():
    wl = make(CONFIGS[1])
    assert tuple(wl.q.shape) == (2, 1, 16, 576) and wl.q.dtype == torch.bfloat16
    assert wl.seqlens.tolist() == [64, 100]
    assert wl.block_table.shape[1] >= 7
    wl4 = make(dataclasses.replace(CONFIGS[4], batch=2))
    assert tuple(wl4.q.shape) == (2, 4, 64, 512) and wl4.sink.shape == (64,)
    assert wl4.nope_codes.shape[1] == 448
    sc = wl4.scale_codes.numpy()
    assert sc[:, :7].min() >= 123 and sc[:, :7].max() <= 131 and np.all(sc[:, 7] == 0)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_device_draw_layout(spec):
    """make_on_device (timing workloads) fills the same paged layout as make(): every logical row
    written (no poison read back), fp8 exponents in range, every other byte 0xFF."""
    from workloads import make_on_device
    wl = make_on_device(spec, "cpu")
    ref = make(spec)
    assert np.array_equal(wl.seqlens, ref.seqlens)
    assert wl.cache.shape == ref.cache.shape and wl.block_table.shape == ref.block_table.shape
    bt = wl.block_table.numpy()
    used = set()
    for b in range(spec.batch):
        L = int(wl.seqlens[b])
        rows = paging.dense_rows(wl.cache.numpy(), bt, b, L, spec.kv_format, spec.d_qk,
                                 spec.d_rope, spec.page_size)
        assert rows.shape == (L, spec.d_qk) and np.all(np.isfinite(rows))
        used.update(bt[b, :-(-L // spec.page_size)].tolist())
    unused = [p for p in range(wl.num_pages) if p not in used]
    assert len(unused) == spec.spare_pages and np.all(wl.cache.numpy()[unused] == 0xFF)
