"""GPU parity of mla_q_absorb / mla_v_up (through the C ABI) against the absorption oracle, and
the three steps around and through the decode against the expanded MHA form."""

import math

import numpy as np
import pytest
import torch

import mla_harness as H
from oracle import absorb, mha
from workloads import Spec, make

pytestmark = pytest.mark.gpu


def _bf16(shape, g, scale=1.0):
    return (torch.randn(*shape, generator=g, dtype=torch.float64) * scale).to(torch.bfloat16)


def _check(got, want, K):
    """bf16 output of an fp32-accumulated K-term dot product: |err| <= 2^-8 |ref| + 1e-3 rms."""
    got = got.to(torch.float64).numpy()
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 1e-3 * np.sqrt(np.mean(want ** 2))
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3e}"
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 5e-3, rel


@pytest.mark.parametrize("T,Hh,P,L,R", [(64, 128, 128, 512, 64), (1, 128, 128, 512, 64),
                                         (100, 3, 64, 128, 8), (70, 5, 32, 64, 0)])
def test_q_absorb(T, Hh, P, L, R):
    import mla_paged_latent_plan_amd as mla
    g = torch.Generator().manual_seed(T + Hh)
    q_nope = _bf16((T, Hh, P), g)
    q_pe = _bf16((T, Hh, R), g) if R else None
    w_uk = _bf16((Hh, L, P), g, 1 / math.sqrt(P))
    q_out = torch.full((T, Hh, L + R), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"[gpu] q_absorb T={T} H={Hh} P={P} L={L} R={R}", flush=True)
    mla.mla_q_absorb(q_nope.cuda(), None if q_pe is None else q_pe.cuda(), w_uk.cuda(), q_out)
    torch.cuda.synchronize()
    got = q_out.cpu()
    want = absorb.q_absorb(q_nope.to(torch.float64).numpy(), w_uk.to(torch.float64).numpy())
    _check(got[:, :, :L], want, P)
    if R:
        assert torch.equal(got[:, :, L:].view(torch.int16), q_pe.view(torch.int16))


@pytest.mark.parametrize("T,Hh,L,V", [(64, 128, 512, 128), (3, 128, 512, 128), (129, 4, 96, 64)])
def test_v_up(T, Hh, L, V):
    import mla_paged_latent_plan_amd as mla
    g = torch.Generator().manual_seed(7 * T + Hh)
    o = _bf16((T, Hh, L), g)
    w_uv = _bf16((Hh, V, L), g, 1 / math.sqrt(L))
    out = torch.full((T, Hh, V), float("nan"), dtype=torch.bfloat16, device="cuda")
    print(f"[gpu] v_up T={T} H={Hh} L={L} V={V}", flush=True)
    mla.mla_v_up(o.cuda(), w_uv.cuda(), out)
    torch.cuda.synchronize()
    want = absorb.v_up(o.to(torch.float64).numpy(), w_uv.to(torch.float64).numpy())
    _check(out.cpu(), want, L)


def test_absorb_decode_up_equals_expanded_mha():
    """q_absorb -> plan/decode/combine -> v_up on the GPU against the expanded MHA form (per-head
    up-projected keys and values, fp64) of the same bf16 inputs: 16 heads of DeepSeek-V3 shape."""
    import mla_paged_latent_plan_amd as mla
    Hh, P, R, L, V = 16, 128, 64, 512, 128
    spec = Spec("absorb_e2e", batch=2, q_len=1, num_heads=Hh, page_size=64, seqlens=(77, 300),
                sm_scale=1 / math.sqrt(P + R), seed=51)
    wl = make(spec)
    g = torch.Generator().manual_seed(52)
    B = spec.batch
    q_nope = _bf16((B, Hh, P), g)
    q_pe = _bf16((B, Hh, R), g)
    w_uk = _bf16((Hh, L, P), g, 1 / math.sqrt(P))
    w_uv = _bf16((Hh, V, L), g, 1 / math.sqrt(L))
    q = torch.empty(B, 1, Hh, L + R, dtype=torch.bfloat16, device="cuda")
    print("[gpu] absorb -> decode -> up", flush=True)
    mla.mla_q_absorb(q_nope.cuda(), q_pe.cuda(), w_uk.cuda(), q)
    torch.cuda.synchronize()
    wl.q = q.cpu()
    out, lse, _, _ = H.run_gpu(wl)
    o_up = torch.empty(B, Hh, V, dtype=torch.bfloat16, device="cuda")
    mla.mla_v_up(out.cuda().reshape(B, Hh, L), w_uv.cuda(), o_up)
    torch.cuda.synchronize()
    W_UK = np.transpose(w_uk.to(torch.float64).numpy(), (1, 0, 2))   # (L, N, P)
    W_UV = np.transpose(w_uv.to(torch.float64).numpy(), (2, 0, 1))   # (L, N, V)
    for b in range(B):
        rows = H.dense_rows(wl, b)
        Lb = int(wl.seqlens[b])
        o_ref, lse_ref = mha.expanded_attention(
            q_nope[b:b + 1].to(torch.float64).numpy(), q_pe[b:b + 1].to(torch.float64).numpy(),
            rows[:, :L], rows[:, L:], W_UK, W_UV, spec.sm_scale, [list(range(Lb))])
        got = o_up[b].cpu().to(torch.float64).numpy()
        rel = np.linalg.norm(got - o_ref[0]) / np.linalg.norm(o_ref[0])
        print(f"[gpu]   request {b}: rel_l2 {rel:.2e}", flush=True)
        # the decode's query is rounded to bf16 after absorption, its output before the up-projection
        assert rel <= 5e-3, rel
        assert np.max(np.abs(lse[b, :, 0].numpy() - lse_ref[:, 0])) <= 2e-2
