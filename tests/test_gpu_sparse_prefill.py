"""GPU parity of the sparse prefill (mla_sparse_prefill through the C ABI) against the oracle."""


import numpy as np
import pytest
import torch

import mla_paged_latent_plan_amd as mla
from mla_harness import LSE_ABS, assert_parity, metrics
from oracle.sparse_prefill import sparse_prefill as oracle_sparse_prefill
from workloads import gen

pytestmark = pytest.mark.gpu

S = gen.SparsePrefillSpec
CASES = [
    # several 64-head tiles, ragged topk, padded early tokens, invalid entries, empty tokens
    S("v3_h128", s_q=37, num_heads=128, s_kv=1500, topk=1000, invalid_frac=0.05, empty_tokens=2,
      seed=11),
    # DSV4 rows, one 64-head tile, long lists split over several work units (combine path)
    S("v4_h64_split", s_q=6, num_heads=64, s_kv=9000, topk=6000, d_qk=512,
      sm_scale=1.0 / np.sqrt(512.0), seed=12),
    # fewer heads than a tile (rows past H repeat the last head), ragged everything
    S("v3_h16", s_q=9, num_heads=16, s_kv=777, topk=200, invalid_frac=0.2, seed=13),
    # heads not a multiple of 64, one valid entry per token at the smallest topk
    S("v3_h100_topk1", s_q=50, num_heads=100, s_kv=300, topk=1, seed=14),
    # a token list of one row past a tile boundary, many splits per token
    S("v3_h128_many_splits", s_q=2, num_heads=128, s_kv=40000, topk=20000, invalid_frac=0.01,
      seed=15),
]


def run(spec, num_cus=None, dev=None):
    q, kv, idx = dev if dev is not None else gen.make_sparse_prefill(spec)
    cus = num_cus or mla.device_num_cus()
    qd, kvd, idd = q.cuda(), kv.cuda(), idx.cuda()
    ws = torch.empty(mla.sparse_prefill_workspace_size(spec.s_q, spec.num_heads, spec.d_qk,
                                                       spec.topk, spec.s_kv, cus),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # stale workspace contents must not matter
    out = torch.full((spec.s_q, spec.num_heads, 512), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    mlog = torch.full((spec.num_heads, spec.s_q), float("nan"), device="cuda")
    lse = torch.full((spec.num_heads, spec.s_q), float("nan"), device="cuda")
    mla.mla_sparse_prefill(qd, kvd, idd, spec.sm_scale, ws, out, mlog, lse, cus)
    torch.cuda.synchronize()
    return (q, kv, idx), out.cpu(), mlog.cpu(), lse.cpu()


def check(spec, out, mlog, lse, inputs, tokens=None):
    q, kv, idx = inputs
    O_ref, M_ref, L_ref, A_ref = oracle_sparse_prefill(q.float().numpy(), kv.float().numpy(),
                                                       idx.numpy(), spec.sm_scale, tokens=tokens,
                                                       abs_mass=True)
    sel = slice(None) if tokens is None else list(tokens)
    o = out[sel]
    l = lse[:, sel]
    m = mlog[:, sel].double().numpy()
    assert_parity(metrics(o, l, O_ref, L_ref, A_ref), ctx=spec.name)
    empty = np.isneginf(M_ref)
    assert np.array_equal(np.isneginf(m), empty), f"{spec.name}: -inf max_logits differ"
    if (~empty).any():
        err = float(np.max(np.abs(m[~empty] - M_ref[~empty])))
        assert err <= LSE_ABS, f"{spec.name}: max_logits error {err}"
    # empty tokens: exact zeros and -inf
    for t in np.nonzero(empty.all(axis=0))[0]:
        assert torch.all(o[t] == 0)


@pytest.mark.parametrize("spec", CASES, ids=[c.name for c in CASES])
def test_sparse_prefill_parity(spec):
    print(f"[sparse_prefill] {spec}", flush=True)
    inputs, out, mlog, lse = run(spec)
    check(spec, out, mlog, lse, inputs)


def test_sparse_prefill_plan_cus_independent():
    """Other work-unit counts split the lists differently; results stay within the bar."""
    spec = CASES[1]
    inputs = gen.make_sparse_prefill(spec)
    for cus in (8, 77):
        print(f"[sparse_prefill] {spec.name} num_cus={cus}", flush=True)
        _, out, mlog, lse = run(spec, num_cus=cus, dev=inputs)
        check(spec, out, mlog, lse, inputs)


def test_sparse_prefill_full_size_sampled():
    """The benchmarked workload (4096 tokens, 128 heads, top-k 2048 of 32768 rows), checked on a
    sample of tokens the oracle computes one by one, plus properties of every row."""
    spec = gen.SPARSE_PREFILL["dsv32_prefill"]
    print(f"[sparse_prefill] {spec}", flush=True)
    inputs, out, mlog, lse = run(spec)
    toks = [0, 1, 777, 2048, 3000, spec.s_q - 1]
    check(spec, out, mlog, lse, inputs, tokens=toks)
    m, l = mlog.double(), lse.double()
    assert torch.isfinite(out.float()).all() and torch.isfinite(m).all() and torch.isfinite(l).all()
    gap = l - m  # 0 <= LSE - max <= ln(topk) (every list holds topk distinct valid rows)
    assert float(gap.min()) >= -LSE_ABS and float(gap.max()) <= np.log(spec.topk) + LSE_ABS


def test_sparse_prefill_graph_replay_matches_eager():
    """The whole call (metadata fill, plan, decode, combine) captured in a HIP graph: every replay
    equals the eager result bitwise, with the outputs and the workspace overwritten by eager work
    between replays (the call rebuilds its metadata and plan on every run)."""
    spec = CASES[1]  # multi-split tokens: partials, split maxima and the combine
    q, kv, idx = gen.make_sparse_prefill(spec)
    cus = mla.device_num_cus()
    qd, kvd, idd = q.cuda(), kv.cuda(), idx.cuda()
    ws = torch.empty(mla.sparse_prefill_workspace_size(spec.s_q, spec.num_heads, spec.d_qk,
                                                       spec.topk, spec.s_kv, cus),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(spec.s_q, spec.num_heads, 512, dtype=torch.bfloat16, device="cuda")
    mlog = torch.empty(spec.num_heads, spec.s_q, device="cuda")
    lse = torch.empty(spec.num_heads, spec.s_q, device="cuda")
    print("[sparse_prefill] graph replay: eager", flush=True)
    mla.mla_sparse_prefill(qd, kvd, idd, spec.sm_scale, ws, out, mlog, lse, cus)
    torch.cuda.synchronize()
    ref = (out.clone(), mlog.clone(), lse.clone())
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        mla.mla_sparse_prefill(qd, kvd, idd, spec.sm_scale, ws, out, mlog, lse, cus, stream=cap)
    torch.cuda.synchronize()
    for k in range(4):
        out.fill_(float("nan"))
        mlog.fill_(0.0)
        lse.fill_(0.0)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        print(f"[sparse_prefill] graph replay {k}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"replay {k}: out"
        assert torch.equal(mlog, ref[1]), f"replay {k}: max_logits"
        assert torch.equal(lse, ref[2]), f"replay {k}: lse"


def test_sparse_prefill_maximum_tokens():
    """8192 tokens, the most one call takes (the plan's per-group state lives in LDS)."""
    spec = S("max_tokens", s_q=8192, num_heads=16, s_kv=9000, topk=64, invalid_frac=0.1, seed=16)
    print(f"[sparse_prefill] {spec}", flush=True)
    inputs, out, mlog, lse = run(spec)
    check(spec, out, mlog, lse, inputs, tokens=[0, 1, 63, 64, 4095, 8190, 8191])
    assert torch.isfinite(out.float()).all()
