"""mla_decode_noalloc (plan and split partials in the library's static device scratch) against the
same decode step through mla_decode_plan, mla_decode and mla_combine with caller buffers: the
outputs must be equal bit for bit (same kernels, same plan), and within the parity bar of the
oracle. Three calls in a row, each smaller than the one before, so a call that read anything a
previous call left in the scratch would show."""

import math

import numpy as np
import pytest
import torch

from workloads import Spec, make

import mla_harness as H

pytestmark = pytest.mark.gpu

S = 1.0 / math.sqrt(192.0)

CALLS = [
    Spec("noalloc_h128", batch=6, q_len=1, num_heads=128, page_size=64,
         seqlens=(1, 63, 64, 65, 700, 2001), sm_scale=S, seed=91),
    Spec("noalloc_h128_small", batch=3, q_len=1, num_heads=128, page_size=64,
         seqlens=(65, 300, 1000), sm_scale=S, seed=92),
    Spec("noalloc_fp8_verify", batch=2, q_len=4, num_heads=16, d_qk=512, kv_format="fp8",
         page_size=64, seqlens=(131, 700), causal=True, window=128, sink=True,
         sm_scale=1 / math.sqrt(512), seed=93),
]


def test_noalloc_matches_caller_buffers():
    import mla_paged_latent_plan_amd as mla
    cus = mla.device_num_cus()
    for spec in CALLS:
        wl = make(spec)
        dev = H.to_device(wl)
        p = H.problem_of(wl, mla)
        print(f"[gpu] noalloc {spec.name}", flush=True)
        ref_out, ref_lse, _, _ = H.run_gpu(wl, cus, dev)
        out = torch.full((spec.batch, spec.q_len, spec.num_heads, spec.d_v), float("nan"),
                         dtype=torch.bfloat16, device="cuda")
        lse = torch.full((spec.batch, spec.num_heads, spec.q_len), float("nan"), device="cuda")
        mla.mla_decode_noalloc(p, cus, dev.q, dev.cache, dev.block_table, dev.seqlens,
                               dev.topk_lens, spec.sm_scale, dev.indices, dev.sink, out, lse)
        torch.cuda.synchronize()
        out, lse = out.cpu(), lse.cpu()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), spec.name
        assert torch.equal(lse, ref_lse), spec.name
        O, L, A = H.oracle_of(wl, abs_mass=True)
        m = H.metrics(out, lse, O, L, A)
        print(f"[gpu]   {m}", flush=True)
        H.assert_parity(m, ctx=spec.name, scaled=H.scaled_bound(wl))
