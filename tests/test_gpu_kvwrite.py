"""GPU parity of mla_kv_write (through the C ABI) against the cache-write oracle: byte-exact.

Where a float decides a byte (the e4m3 code, the scale exponent), both sides decide it on the
same exact value: x * 2^-k of a bf16 x is exact in fp32 and in float64."""

import math

import numpy as np
import pytest
import torch

from oracle import kvwrite
from workloads import CONFIGS, make
from workloads.gen import cache_layout

pytestmark = pytest.mark.gpu


def _rows(n, d_nope, d_rope, seed):
    """bf16 rows with a different magnitude per 64-value group, plus special groups."""
    g = torch.Generator().manual_seed(seed)
    kv = torch.randn(n, d_nope, generator=g, dtype=torch.float64)
    e = torch.randint(-24, 25, (n, d_nope // 64), generator=g).repeat_interleave(64, dim=1)
    kv = kv * torch.pow(2.0, e.to(torch.float64))
    if n >= 8:
        kv[0, :64] = 0.0                                  # all-zero group
        kv[0, 64:128] = -0.0                              # negative zeros
        kv[1, :64] = torch.linspace(-448, 448, 64)        # amax exactly 448: scale 1
        kv[1, 64:128] = torch.linspace(-1, 1, 64) * 448 * 2.0 ** 5
        kv[2, :64] *= 2.0 ** -100                         # tiny values
        kv[2, 64:128] = 3.0
        kv[2, 64] = 3.0 * 2.0 ** -20                      # below half the smallest subnormal
        kv[2, 65] = -3.0 * 2.0 ** -20                     #   (scale 2^-7): signed zeros
        kv[2, 66] = 2.0 ** -17                            # exactly half of it: tie, code 0
        kv[2, 67] = 3.0 * 2.0 ** -18                      # 1.5 halves: rounds up to code 1
        # midpoints between e4m3 neighbours at scale 1 (amax 448 in the group): ties to even
        mags = [kvwrite._MAGS[i] for i in range(len(kvwrite._MAGS))]
        mids = [(a + b) / 2 for a, b in zip(mags[:-1], mags[1:])]
        kv[3, :63] = torch.tensor(mids[-63:], dtype=torch.float64)
        kv[3, 63] = 448.0
    kv_c = kv.to(torch.bfloat16)
    k_pe = torch.randn(n, d_rope, generator=g).to(torch.bfloat16)
    return kv_c, k_pe


def _run(fmt, d_qk, page_size, num_pages, slots, seed):
    import mla_paged_latent_plan_amd as mla
    d_rope = 64
    lay = cache_layout(fmt, d_qk, d_rope, page_size)
    stride = lay["page_stride"]
    n = len(slots)
    kv_c, k_pe = _rows(n, d_qk - d_rope, d_rope, seed)
    cache = torch.full((num_pages, stride), 0xFF, dtype=torch.uint8)
    p = mla.make_problem(1, 1, 16, d_qk, mla.MLA_KV_BF16 if fmt == "bf16" else mla.MLA_KV_FP8,
                         page_size, stride, num_pages, 1)
    dev_cache = cache.cuda()
    print(f"[gpu] kv_write {fmt} d_qk={d_qk} page={page_size} n={n}", flush=True)
    mla.mla_kv_write(p, kv_c.cuda(), k_pe.cuda(), torch.tensor(slots, dtype=torch.int64).cuda(),
                     dev_cache)
    torch.cuda.synchronize()
    return cache, dev_cache.cpu(), kv_c, k_pe


@pytest.mark.parametrize("fmt,d_qk,page_size", [("fp8", 576, 64), ("fp8", 512, 64),
                                                ("bf16", 576, 16), ("bf16", 512, 64),
                                                ("fp8", 576, 1)])
def test_kv_write_bytes_exact(fmt, d_qk, page_size):
    num_pages = 9
    total = num_pages * page_size
    g = np.random.default_rng(page_size + d_qk)
    n = min(200, total)
    slots = g.permutation(total)[:n].astype(np.int64)
    slots[5] = -1                 # no slot: skipped
    slots[6] = total + 3          # outside the cache: skipped
    before, got, kv_c, k_pe = _run(fmt, d_qk, page_size, num_pages, slots, seed=n + d_qk)
    want = kvwrite.write_rows(before.numpy(), fmt, page_size, kv_c.to(torch.float64).numpy(),
                              k_pe.to(torch.float64).numpy(), slots)
    diff = np.argwhere(got.numpy() != want)
    assert diff.size == 0, f"{len(diff)} bytes differ, first at {diff[:4].tolist()}"


def test_kv_write_no_tokens_is_a_no_op():
    before, got, _, _ = _run("fp8", 576, 64, 2, np.zeros(0, dtype=np.int64), seed=1)
    assert torch.equal(before, got)


def test_kv_write_full_size_sampled():
    """Every row of the fp8 DeepSeek-V3 workload (64 requests, lengths U[1024, 8192], pages of 64)
    written in one launch, in request order through the block table; a sample of rows compared
    byte for byte with the oracle, and the untouched spare pages unchanged."""
    import mla_paged_latent_plan_amd as mla
    wl = make(CONFIGS[3])
    s = wl.spec
    lay = cache_layout("fp8", s.d_qk, s.d_rope, s.page_size)
    bt = wl.block_table.numpy()
    L = wl.seqlens.astype(np.int64)
    req = np.repeat(np.arange(s.batch), L)
    pos = np.concatenate([np.arange(x) for x in L])
    slots = bt[req, pos // s.page_size].astype(np.int64) * s.page_size + pos % s.page_size
    n = len(slots)
    g = torch.Generator().manual_seed(303)
    kv_c = torch.randn(n, s.d_qk - s.d_rope, generator=g).to(torch.bfloat16)
    k_pe = torch.randn(n, s.d_rope, generator=g).to(torch.bfloat16)
    p = mla.make_problem(s.batch, 1, s.num_heads, s.d_qk, mla.MLA_KV_FP8, s.page_size,
                         wl.page_stride, wl.num_pages, int(bt.shape[1]))
    cache = torch.full_like(wl.cache, 0xFF).cuda()
    print(f"[gpu] kv_write full size: {n} rows", flush=True)
    mla.mla_kv_write(p, kv_c.cuda(), k_pe.cuda(), torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    rb = lay["row_bytes"]
    sample = np.random.default_rng(4).choice(n, 400, replace=False)
    for i in sample:
        row, slot = kvwrite.encode_row(kv_c[i].to(torch.float64).numpy(),
                                       k_pe[i].to(torch.float64).numpy(), "fp8")
        page, r = divmod(int(slots[i]), s.page_size)
        assert np.array_equal(got[page, r * rb:(r + 1) * rb], row), f"row {i}"
        off = lay["scale_offset"] + 8 * r
        assert np.array_equal(got[page, off:off + 8], slot), f"scale slot {i}"
    used = np.unique(slots // s.page_size)
    spare = np.setdiff1d(np.arange(wl.num_pages), used)
    assert spare.size > 0 and np.all(got[spare] == 0xFF)
