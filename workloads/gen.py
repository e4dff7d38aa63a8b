"""Seeded synthetic MLA decode workloads and the paged cache byte layout.

Shapes follow the MLA pages: DeepSeek-V3 latent rows are 576 wide (512 latent + 64 RoPE,
vLLM mla_attention.py module docstring, "Data-Movement Friendly Approach"); DeepSeek-V4 rows are
512 wide (448 NoPE + 64 RoPE, HALOps MLA API, mla_attention). The fp8 page layout follows the
HALOps kv_cache description (rows of e4m3 NoPE bytes followed by a bf16 RoPE tail, then one 8-byte
ue8m0 scale slot per row after the rows); for 576-wide rows the same layout is used with 512 NoPE
bytes, i.e. 640-byte rows.

Nothing here computes attention: values are drawn, cast to the storage dtype by torch, and copied
into pages. Unused pages, unused tail slots and padding bytes are filled with 0xFF, which is NaN in
bf16, e4m3fn and ue8m0, so any read of them shows up in the outputs.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np
import torch

SCALE_SLOT_BYTES = 8
BLOCK_ROWS = 64


def cache_layout(kv_format: str, d_qk: int, d_rope: int, page_size: int) -> dict:
    """Byte layout of one cache page.

    bf16: page_size rows of d_qk bfloat16 values.
    fp8:  page_size rows of [d_qk - d_rope e4m3 bytes][d_rope bfloat16], then page_size 8-byte
          scale slots (one ue8m0 byte per 64 NoPE values, zero padded); the default page stride is
          rounded up to a multiple of the row size.
    """
    if kv_format == "bf16":
        row_bytes = 2 * d_qk
        return dict(d_nope=d_qk - d_rope, row_bytes=row_bytes, scale_offset=None,
                    page_stride=page_size * row_bytes)
    if kv_format == "fp8":
        d_nope = d_qk - d_rope
        row_bytes = d_nope + 2 * d_rope
        raw = page_size * (row_bytes + SCALE_SLOT_BYTES)
        stride = -(-raw // row_bytes) * row_bytes
        return dict(d_nope=d_nope, row_bytes=row_bytes, scale_offset=page_size * row_bytes,
                    page_stride=stride)
    raise ValueError(f"unknown kv_format {kv_format!r}")


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    q_len: int
    num_heads: int
    d_qk: int = 576
    d_v: int = 512
    d_rope: int = 64
    kv_format: str = "bf16"
    page_size: int = 64
    seqlens: Optional[Tuple[int, ...]] = None
    len_range: Optional[Tuple[int, int]] = None
    sm_scale: float = 1.0 / math.sqrt(192.0)
    causal: bool = False
    window: int = 0
    topk: int = 0
    sink: bool = False
    scale_exp_range: Tuple[int, int] = (-4, 4)
    seed: int = 0
    plan_cus: Optional[int] = None     # compute units the plan spreads over (None: the device's)
    spare_pages: int = 2
    poison: bool = True
    page_seed: Optional[int] = None    # separate seed for the page permutation (None: the main one)

    @property
    def rows_per_group(self) -> int:
        return self.num_heads if self.topk > 0 else self.q_len * self.num_heads


# The five workloads the MLA decode path is measured on.
CONFIGS = {
    1: Spec("tiny", batch=2, q_len=1, num_heads=16, d_qk=576, page_size=16, seqlens=(64, 100),
            sm_scale=1.0 / math.sqrt(576.0), seed=1001, plan_cus=2),
    2: Spec("dsv3_bf16", batch=64, q_len=1, num_heads=128, d_qk=576, page_size=64,
            len_range=(1024, 8192), sm_scale=1.0 / math.sqrt(192.0), seed=1002),
    3: Spec("dsv3_fp8", batch=64, q_len=1, num_heads=128, d_qk=576, kv_format="fp8", page_size=64,
            len_range=(1024, 8192), sm_scale=1.0 / math.sqrt(192.0), seed=1003),
    4: Spec("dsv4_verify", batch=32, q_len=4, num_heads=64, d_qk=512, kv_format="fp8",
            page_size=64, len_range=(1024, 8192), sm_scale=1.0 / math.sqrt(512.0), causal=True,
            window=128, sink=True, seed=1004),
    5: Spec("long_sparse", batch=4, q_len=1, num_heads=128, d_qk=576, page_size=64,
            seqlens=(131072,) * 4, sm_scale=1.0 / math.sqrt(192.0), topk=2048, seed=1005),
}

# Labelled extra shapes that show the bandwidth-bound regime the small workloads cannot.
SUPPLEMENTARY = {
    "s1": dataclasses.replace(CONFIGS[2], name="dsv3_bf16_h16", num_heads=16, seed=1012),
    "s4": dataclasses.replace(CONFIGS[4], name="dsv4_verify_b512", batch=512, seed=1014),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    seqlens: np.ndarray            # int32 [B]
    q: torch.Tensor                # bf16 [B, Sq, H, d_qk]
    row_offsets: np.ndarray        # int64 [B + 1]: logical rows of request b are [off[b], off[b+1])
    rows_bf16: Optional[torch.Tensor]    # bf16 [total, d_qk]           (kv_format bf16)
    nope_codes: Optional[torch.Tensor]   # uint8 [total, d_nope] e4m3   (kv_format fp8)
    scale_codes: Optional[torch.Tensor]  # uint8 [total, 8] ue8m0 slot  (kv_format fp8)
    rope_bf16: Optional[torch.Tensor]    # bf16 [total, d_rope]         (kv_format fp8)
    cache: torch.Tensor            # uint8 [num_pages, page_stride]
    block_table: torch.Tensor      # int32 [B, max_pages]
    page_stride: int
    indices: Optional[torch.Tensor]      # int32 [B, Sq, topk]
    topk_lens: Optional[torch.Tensor]    # int32 [B * Sq]
    sink: Optional[torch.Tensor]         # fp32 [H]

    @property
    def num_pages(self) -> int:
        return int(self.cache.shape[0])

    def request_rows(self, b: int):
        """Logical rows of request b in their storage dtypes (views, no copy)."""
        a, e = int(self.row_offsets[b]), int(self.row_offsets[b + 1])
        if self.spec.kv_format == "bf16":
            return self.rows_bf16[a:e]
        return self.nope_codes[a:e], self.scale_codes[a:e], self.rope_bf16[a:e]


def _draw_seqlens(spec: Spec, g: torch.Generator) -> np.ndarray:
    if spec.seqlens is not None:
        assert len(spec.seqlens) == spec.batch
        return np.asarray(spec.seqlens, dtype=np.int32)
    lo, hi = spec.len_range
    return torch.randint(lo, hi + 1, (spec.batch,), generator=g).numpy().astype(np.int32)


def make(spec: Spec, seqlens: Optional[np.ndarray] = None,
         topk_lens: Optional[np.ndarray] = None) -> Workload:
    """Draw the workload of `spec` from its seed (CPU tensors)."""
    g = torch.Generator().manual_seed(spec.seed)
    if seqlens is None:
        seqlens = _draw_seqlens(spec, g)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    B, Sq, H, dqk, dr = spec.batch, spec.q_len, spec.num_heads, spec.d_qk, spec.d_rope
    lay = cache_layout(spec.kv_format, dqk, dr, spec.page_size)
    ps, row_bytes, stride = spec.page_size, lay["row_bytes"], lay["page_stride"]

    q = torch.randn(B, Sq, H, dqk, generator=g).to(torch.bfloat16)
    lens = np.maximum(seqlens.astype(np.int64), 0)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    total = int(off[-1])

    rows_bf16 = nope = scales = rope = None
    if spec.kv_format == "bf16":
        rows_bf16 = torch.randn(total, dqk, generator=g).to(torch.bfloat16)
    else:
        d_nope = lay["d_nope"]
        ngrp = -(-d_nope // 64)
        nope = torch.randn(total, d_nope, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
        lo, hi = spec.scale_exp_range
        exps = torch.randint(lo, hi + 1, (total, ngrp), generator=g)
        scales = torch.zeros(total, SCALE_SLOT_BYTES, dtype=torch.uint8)
        scales[:, :ngrp] = (127 + exps).to(torch.uint8)
        rope = torch.randn(total, dr, generator=g).to(torch.bfloat16)

    # Pages: each request owns ceil(L/ps) logical pages; physical ids are a random permutation.
    npages_req = (lens + ps - 1) // ps
    poff = np.zeros(B + 1, dtype=np.int64)
    poff[1:] = np.cumsum(npages_req)
    num_pages = int(poff[-1]) + spec.spare_pages
    pg = g if spec.page_seed is None else torch.Generator().manual_seed(spec.page_seed)
    perm = torch.randperm(num_pages, generator=pg).numpy().astype(np.int64)
    max_pages = int(npages_req.max(initial=0)) + 1
    spare_phys = perm[int(poff[-1])] if spec.spare_pages > 0 else perm[0]
    block_table = np.full((B, max_pages), spare_phys, dtype=np.int32)
    for b in range(B):
        n = int(npages_req[b])
        block_table[b, :n] = perm[poff[b]:poff[b] + n]

    # torch's fill: numpy's takes seconds per hundred MB here
    cache_t = torch.full((num_pages, stride), 0xFF if spec.poison else 0, dtype=torch.uint8)
    cache = cache_t.numpy()
    if total > 0:
        req = np.repeat(np.arange(B), lens)
        pos = np.arange(total, dtype=np.int64) - off[req]
        phys = perm[poff[req] + pos // ps]
        slot = pos % ps
        rview = np.lib.stride_tricks.as_strided(cache, shape=(num_pages, ps, row_bytes),
                                                strides=(stride, row_bytes, 1))
        if spec.kv_format == "bf16":
            rview[phys, slot] = rows_bf16.view(torch.uint8).numpy().reshape(total, row_bytes)
        else:
            d_nope = lay["d_nope"]
            rview[phys, slot, :d_nope] = nope.numpy()
            rview[phys, slot, d_nope:] = rope.view(torch.uint8).numpy().reshape(total, 2 * dr)
            sview = np.lib.stride_tricks.as_strided(
                cache[:, lay["scale_offset"]:], shape=(num_pages, ps, SCALE_SLOT_BYTES),
                strides=(stride, SCALE_SLOT_BYTES, 1))
            sview[phys, slot] = scales.numpy()

    indices = None
    if spec.topk > 0:
        idx = np.full((B, Sq, spec.topk), -1, dtype=np.int32)
        for b in range(B):
            for t in range(Sq):
                L = int(lens[b])
                k = min(L, spec.topk)
                if k > 0:
                    idx[b, t, :k] = torch.randperm(L, generator=g)[:k].numpy()
        indices = torch.from_numpy(idx)
    tl = None if topk_lens is None else torch.from_numpy(np.asarray(topk_lens, dtype=np.int32))
    sink = torch.randn(H, generator=g, dtype=torch.float32) if spec.sink else None

    return Workload(spec=spec, seqlens=seqlens, q=q, row_offsets=off, rows_bf16=rows_bf16,
                    nope_codes=nope, scale_codes=scales, rope_bf16=rope,
                    cache=cache_t, block_table=torch.from_numpy(block_table),
                    page_stride=stride, indices=indices, topk_lens=tl, sink=sink)



def make_on_device(spec: Spec, device) -> Workload:
    """The workload of `spec` drawn on `device`, for timing only.

    Same recipe as make(): the same request lengths, a random page permutation, values N(0, 1)
    cast to the storage dtype, ue8m0 exponents uniform in the spec's range, top-k lists drawn
    without replacement, 0xFF in every byte no row owns. The values come from the device's
    generator, so they differ from make()'s (which the oracle reads); the logical row tensors are
    not kept. Drawing a multi-GB cache this way takes milliseconds instead of a minute of host
    time."""
    g = torch.Generator().manual_seed(spec.seed)
    seqlens = _draw_seqlens(spec, g)
    gd = torch.Generator(device=device).manual_seed(spec.seed)
    B, Sq, H, dqk, dr = spec.batch, spec.q_len, spec.num_heads, spec.d_qk, spec.d_rope
    lay = cache_layout(spec.kv_format, dqk, dr, spec.page_size)
    ps, row_bytes, stride = spec.page_size, lay["row_bytes"], lay["page_stride"]
    q = torch.randn(B, Sq, H, dqk, generator=gd, device=device).to(torch.bfloat16)
    lens = np.maximum(seqlens.astype(np.int64), 0)
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    total = int(off[-1])
    npages_req = (lens + ps - 1) // ps
    poff = np.zeros(B + 1, dtype=np.int64)
    poff[1:] = np.cumsum(npages_req)
    num_pages = int(poff[-1]) + spec.spare_pages
    perm = torch.randperm(num_pages, generator=g).numpy().astype(np.int64)
    max_pages = int(npages_req.max(initial=0)) + 1
    spare_phys = perm[int(poff[-1])] if spec.spare_pages > 0 else perm[0]
    block_table = np.full((B, max_pages), spare_phys, dtype=np.int32)
    for b in range(B):
        n = int(npages_req[b])
        block_table[b, :n] = perm[poff[b]:poff[b] + n]
    cache = torch.full((num_pages, stride), 0xFF if spec.poison else 0, dtype=torch.uint8, device=device)
    if total > 0:
        req = np.repeat(np.arange(B), lens)
        pos = np.arange(total, dtype=np.int64) - off[req]
        phys = torch.from_numpy(perm[poff[req] + pos // ps]).to(device)
        slot = torch.from_numpy(pos % ps).to(device)
        rview = cache.as_strided((num_pages, ps, row_bytes), (stride, row_bytes, 1))
        chunk = 1 << 18  # rows per draw: bounds the fp32 temporaries
        for a in range(0, total, chunk):
            e = min(total, a + chunk)
            ph, sl = phys[a:e], slot[a:e]
            if spec.kv_format == "bf16":
                rows = torch.randn(e - a, dqk, generator=gd, device=device).to(torch.bfloat16)
                rview[ph, sl] = rows.view(torch.uint8).reshape(e - a, row_bytes)
            else:
                d_nope = lay["d_nope"]
                ngrp = -(-d_nope // 64)
                nope = torch.randn(e - a, d_nope, generator=gd, device=device).to(torch.float8_e4m3fn)
                rope = torch.randn(e - a, dr, generator=gd, device=device).to(torch.bfloat16)
                rv = rview[ph, sl]
                rv[:, :d_nope] = nope.view(torch.uint8)
                rv[:, d_nope:] = rope.view(torch.uint8).reshape(e - a, 2 * dr)
                rview[ph, sl] = rv
                lo, hi = spec.scale_exp_range
                exps = torch.randint(lo, hi + 1, (e - a, ngrp), generator=gd, device=device)
                sc = torch.zeros(e - a, SCALE_SLOT_BYTES, dtype=torch.uint8, device=device)
                sc[:, :ngrp] = (127 + exps).to(torch.uint8)
                sview = cache[:, lay["scale_offset"]:].as_strided(
                    (num_pages, ps, SCALE_SLOT_BYTES), (stride, SCALE_SLOT_BYTES, 1))
                sview[ph, sl] = sc
    indices = None
    if spec.topk > 0:
        idx = torch.full((B, Sq, spec.topk), -1, dtype=torch.int32, device=device)
        for b in range(B):
            for t in range(Sq):
                L = int(lens[b])
                k = min(L, spec.topk)
                if k > 0:
                    idx[b, t, :k] = torch.randperm(L, generator=gd, device=device)[:k].to(torch.int32)
        indices = idx
    sink = torch.randn(H, generator=gd, device=device, dtype=torch.float32) if spec.sink else None
    return Workload(spec=spec, seqlens=seqlens, q=q, row_offsets=off, rows_bf16=None,
                    nope_codes=None, scale_codes=None, rope_bf16=None, cache=cache,
                    block_table=torch.from_numpy(block_table).to(device), page_stride=stride,
                    indices=indices, topk_lens=None, sink=sink)

# ---- sparse prefill (FlashMLA wrapper, flash_mla_sparse_fwd) ----------------------------------

@dataclasses.dataclass
class SparsePrefillSpec:
    """Prefill tokens attending over index lists into one flat latent buffer kv [s_kv, d_qk].

    Token t sits at position s_kv - s_q + t (the prefill's tokens are the buffer's last rows) and
    lists topk rows of its causal prefix [0, pos_t]: the whole prefix, padded with -1, when it has
    at most topk rows, else topk distinct rows spread over it (a sorted uniform draw, columns then
    shuffled by one permutation shared by all tokens). `invalid_frac` of the remaining entries are
    replaced by -1 or by rows past s_kv, and the first `empty_tokens` tokens list no valid row.
    """
    name: str
    s_q: int
    num_heads: int
    s_kv: int
    topk: int
    d_qk: int = 576
    sm_scale: float = 1.0 / math.sqrt(192.0)
    invalid_frac: float = 0.0
    empty_tokens: int = 0
    seed: int = 0


SPARSE_PREFILL = {
    "dsv32_prefill": SparsePrefillSpec("dsv32_prefill", s_q=4096, num_heads=128, s_kv=32768,
                                       topk=2048, seed=1101),
}


def make_sparse_prefill(spec: SparsePrefillSpec):
    """(q bf16 [s_q, H, d_qk], kv bf16 [s_kv, d_qk], indices int32 [s_q, topk]) on the CPU."""
    g = torch.Generator().manual_seed(spec.seed)
    s_q, H, d, k, n = spec.s_q, spec.num_heads, spec.d_qk, spec.topk, spec.s_kv
    q = torch.randn(s_q, H, d, generator=g).to(torch.bfloat16)
    kv = torch.randn(n, d, generator=g).to(torch.bfloat16)
    pos = torch.arange(s_q, dtype=torch.int64) + (n - s_q)
    avail = (pos + 1).clamp(min=0)                           # rows of each token's prefix
    ar = torch.arange(k, dtype=torch.int64)
    # distinct rows: sorted draws from [0, avail - k] plus 0..k-1
    span = (avail - k).clamp(min=0) + 1
    draw = (torch.rand(s_q, k, generator=g, dtype=torch.float64) * span[:, None].double()).long()
    draw = torch.sort(draw, dim=1).values + ar[None, :]
    whole = torch.where(ar[None, :] < avail[:, None], ar[None, :], torch.full_like(draw, -1))
    idx = torch.where((avail <= k)[:, None], whole, draw)
    idx = idx[:, torch.randperm(k, generator=g)]
    if spec.invalid_frac > 0:
        hit = torch.rand(s_q, k, generator=g) < spec.invalid_frac
        bad = torch.where(torch.rand(s_q, k, generator=g) < 0.5, torch.full_like(idx, -1),
                          n + torch.randint(0, 1000, (s_q, k), generator=g))
        idx = torch.where(hit, bad, idx)
    if spec.empty_tokens > 0:
        idx[:spec.empty_tokens] = -1
    return q, kv, idx.to(torch.int32).contiguous()
