"""Pins of the context-gather oracle (oracle/gather.py) against the depager (oracle/paging.py)."""

import dataclasses

import numpy as np
import pytest

from oracle import gather, paging
from workloads import Spec, make


@pytest.mark.parametrize("fmt,d_qk", [("bf16", 576), ("fp8", 576), ("fp8", 512)])
def test_gather_equals_depager_spans(fmt, d_qk):
    spec = Spec("g", batch=3, q_len=1, num_heads=16, d_qk=d_qk, kv_format=fmt, page_size=16,
                seqlens=(40, 7, 90), seed=9)
    wl = make(spec)
    cache = wl.cache.numpy()
    bt = wl.block_table.numpy()
    # spans: request 0 rows [5, 40), request 1 rows [0, 7), request 2 rows [16, 80)
    starts = np.array([5, 0, 16], dtype=np.int32)
    lens = np.array([35, 7, 64])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t2s = np.repeat(np.arange(3), lens).astype(np.int32)
    got = gather.gather_context(cache, bt, cu, starts, t2s, fmt, d_qk, 64, 16)
    for r in range(3):
        L = int(wl.seqlens[r])
        dense = paging.dense_rows(cache, bt, r, L, fmt, d_qk, 64, 16)
        np.testing.assert_array_equal(got[cu[r]:cu[r + 1]], dense[starts[r]:starts[r] + lens[r]])


def test_gather_out_of_range_rows_are_zero():
    spec = Spec("g", batch=1, q_len=1, num_heads=16, page_size=16, seqlens=(20,), seed=3)
    wl = make(spec)
    bt = wl.block_table.numpy().copy()
    bt[0, 1] = 10 ** 6  # a page past the cache
    cu = np.array([0, 40], dtype=np.int32)
    got = gather.gather_context(wl.cache.numpy(), bt, cu, None, np.zeros(40, dtype=np.int32),
                                "bf16", 576, 64, 16)
    assert np.all(got[16:32] == 0)           # the missing page
    assert np.all(got[16 * bt.shape[1]:] == 0)  # past the block table
    dense = paging.dense_rows(wl.cache.numpy(), wl.block_table.numpy(), 0, 16, "bf16", 576, 64, 16)
    np.testing.assert_array_equal(got[:16], dense)
