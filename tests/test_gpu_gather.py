"""GPU parity of mla_gather_context (through the C ABI) against the gather oracle: exact values
(bf16 copies, and fp8 values times power-of-two scales, which bf16 holds exactly)."""

import numpy as np
import pytest
import torch

from oracle import gather
from workloads import CONFIGS, Spec, make

pytestmark = pytest.mark.gpu


def _problem(wl, mla):
    s = wl.spec
    return mla.make_problem(s.batch, s.q_len, s.num_heads, s.d_qk,
                            mla.MLA_KV_BF16 if s.kv_format == "bf16" else mla.MLA_KV_FP8,
                            s.page_size, wl.page_stride, wl.num_pages, int(wl.block_table.shape[1]))


def _run(wl, starts, lens, bt=None):
    import mla_paged_latent_plan_amd as mla
    s = wl.spec
    bt = wl.block_table if bt is None else bt
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    t2s = torch.from_numpy(np.repeat(np.arange(len(lens)), lens).astype(np.int32))
    st = None if starts is None else torch.from_numpy(np.asarray(starts, dtype=np.int32))
    n = int(cu[-1])
    dst = torch.full((n, s.d_qk), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"[gpu] gather {s.kv_format} d_qk={s.d_qk} rows={n}", flush=True)
    mla.mla_gather_context(_problem(wl, mla), bt.cuda(), cu.cuda(), None if st is None else st.cuda(),
                           t2s.cuda(), wl.cache.cuda(), dst)
    torch.cuda.synchronize()
    want = gather.gather_context(wl.cache.numpy(), bt.numpy(), cu.numpy(),
                                 None if st is None else st.numpy(), t2s.numpy(), s.kv_format,
                                 s.d_qk, s.d_rope, s.page_size)
    return dst.cpu().to(torch.float64).numpy(), want


@pytest.mark.parametrize("fmt,d_qk,page", [("bf16", 576, 16), ("fp8", 576, 64), ("fp8", 512, 64),
                                            ("bf16", 512, 32)])
def test_gather_exact(fmt, d_qk, page):
    spec = Spec("gather", batch=4, q_len=1, num_heads=16, d_qk=d_qk, kv_format=fmt, page_size=page,
                seqlens=(300, 5, 1000, 64), scale_exp_range=(-6, 6), seed=61)
    wl = make(spec)
    got, want = _run(wl, [17, 0, 256, 0], np.array([283, 5, 700, 64]))
    assert np.array_equal(got, want)


def test_gather_out_of_range_rows_are_zero():
    spec = Spec("gather_oob", batch=2, q_len=1, num_heads=16, page_size=16, seqlens=(40, 40), seed=62)
    wl = make(spec)
    bt = wl.block_table.clone()
    bt[1, 0] = 10 ** 6       # a page past the cache
    got, want = _run(wl, None, np.array([40, 60]), bt)
    # request 1's span runs past its 40 rows: unused slots of its last page hold poison (NaN) on
    # both sides (compared as NaN), entries past them give zero rows
    assert np.array_equal(got, want, equal_nan=True)
    assert np.all(got[40:56] == 0)  # the page past the cache


def test_gather_full_size_fp8():
    """The whole context of the fp8 DeepSeek-V3 workload (64 requests, lengths U[1024, 8192]) in
    one launch; sampled rows against the oracle."""
    import mla_paged_latent_plan_amd as mla
    wl = make(CONFIGS[3])
    s = wl.spec
    lens = wl.seqlens.astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t2s = np.repeat(np.arange(s.batch), lens).astype(np.int32)
    n = int(cu[-1])
    dst = torch.empty((n, s.d_qk), dtype=torch.bfloat16, device="cuda")
    print(f"[gpu] gather full size: {n} rows", flush=True)
    mla.mla_gather_context(_problem(wl, mla), wl.block_table.cuda(), torch.from_numpy(cu).cuda(),
                           None, torch.from_numpy(t2s).cuda(), wl.cache.cuda(), dst)
    torch.cuda.synchronize()
    idx = np.random.default_rng(5).choice(n, 2000, replace=False)
    got = dst.cpu()[torch.from_numpy(idx)].to(torch.float64).numpy()
    # the oracle gathers the sampled rows one by one through their requests
    rows = np.empty((len(idx), s.d_qk))
    for k, i in enumerate(idx):
        r = int(t2s[i])
        one = gather.gather_context(wl.cache.numpy(), wl.block_table.numpy()[r:r + 1],
                                    np.array([0, 1], dtype=np.int32), np.array([i - cu[r]], dtype=np.int32),
                                    np.zeros(1, dtype=np.int32), s.kv_format, s.d_qk, s.d_rope,
                                    s.page_size)
        rows[k] = one[0]
    assert np.array_equal(got, rows)


def test_chunked_context_gather_covers_every_row():
    """Plan the chunks of a set of contexts on the host (workspace 4096 rows, page-aligned splits),
    gather each chunk through the block-table rows of its requests, and check that the chunks
    together reproduce every request's context exactly, in order."""
    import mla_paged_latent_plan_amd as mla
    from oracle import paging
    spec = Spec("chunked", batch=7, q_len=1, num_heads=16, kv_format="fp8", page_size=64,
                seqlens=(3000, 0, 700, 64, 5000, 1, 2500), seed=63)
    wl = make(spec)
    s = spec
    W = 4096
    plan = mla.plan_context_chunks(wl.seqlens, W, s.page_size)
    p = _problem(wl, mla)
    cache_d = wl.cache.cuda()
    got = {r: [] for r in range(s.batch)}
    for ch in plan:
        reqs = [r for r, _, _ in ch]
        # requests in order; those between them have no context rows
        assert all(int(wl.seqlens[x]) == 0 for x in range(reqs[0], reqs[-1] + 1) if x not in reqs)
        lens = np.array([n for _, _, n in ch])
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        starts = torch.tensor([st for _, st, _ in ch], dtype=torch.int32)
        t2s = torch.from_numpy(np.repeat(np.arange(len(ch)), lens).astype(np.int32))
        dst = torch.empty(int(cu[-1]), s.d_qk, dtype=torch.bfloat16, device="cuda")
        mla.mla_gather_context(p, wl.block_table[torch.tensor(reqs)].contiguous().cuda(), cu.cuda(),
                               starts.cuda(), t2s.cuda(), cache_d, dst)
        torch.cuda.synchronize()
        out = dst.cpu().to(torch.float64).numpy()
        for k, (r, st, n) in enumerate(ch):
            got[r].append(out[cu[k]:cu[k] + n])
    print(f"[gpu] chunked gather: {len(plan)} chunks", flush=True)
    for r in range(s.batch):
        L = int(wl.seqlens[r])
        rows = np.concatenate(got[r]) if got[r] else np.zeros((0, s.d_qk))
        want = paging.dense_rows(wl.cache.numpy(), wl.block_table.numpy(), r, L, s.kv_format,
                                 s.d_qk, s.d_rope, s.page_size)
        assert np.array_equal(rows, want), r
