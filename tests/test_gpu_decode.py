"""GPU parity of the HIP path (plan, decode, combine through the C ABI) against the CPU oracle.

Every case runs on seeded synthetic inputs whose unused cache bytes are NaN, so a read outside the
visible rows shows up as a non-finite output."""

import dataclasses
import math

import numpy as np
import pytest
import torch

from workloads import CONFIGS, SUPPLEMENTARY, Spec, make

import mla_harness as H

pytestmark = pytest.mark.gpu

S = 1.0 / math.sqrt(192.0)

CASES = {
    "cfg1_tiny": (CONFIGS[1], None),
    "h128_edges": (Spec("h128_edges", batch=6, q_len=1, num_heads=128, page_size=64,
                        seqlens=(1, 63, 64, 65, 700, 2001), sm_scale=S, seed=11), None),
    "h16_page16": (Spec("h16_page16", batch=7, q_len=1, num_heads=16, page_size=16,
                        seqlens=(0, 1, 15, 130, 511, 1000, 64), sm_scale=S, seed=12), None),
    "h32_page32": (Spec("h32_page32", batch=3, q_len=1, num_heads=32, page_size=32,
                        seqlens=(5, 300, 129), sm_scale=S, seed=13), None),
    "h64_sq2_causal": (Spec("h64_sq2_causal", batch=4, q_len=2, num_heads=64, page_size=64,
                            seqlens=(1, 2, 777, 130), causal=True, sm_scale=S, seed=14), None),
    "h24_odd_heads": (Spec("h24_odd_heads", batch=2, q_len=1, num_heads=24, page_size=64,
                           seqlens=(100, 333), sm_scale=S, seed=18), None),
    "d512_window_sink": (Spec("d512_window_sink", batch=4, q_len=4, num_heads=16, d_qk=512,
                              page_size=64, seqlens=(3, 131, 1000, 4), causal=True, window=128,
                              sink=True, sm_scale=1 / math.sqrt(512), seed=15), None),
    # bf16 rows, d_qk 512 (no RoPE region) at 64-row tiles: 64 heads x 2 causal tokens
    "d512_h64_sq2": (Spec("d512_h64_sq2", batch=3, q_len=2, num_heads=64, d_qk=512, page_size=64,
                          seqlens=(2, 640, 97), causal=True, sm_scale=1 / math.sqrt(512), seed=19),
                     None),
    # 40 stacked rows: one 64-row tile with 24 padding rows
    "h40_padded_tile": (Spec("h40_padded_tile", batch=3, q_len=1, num_heads=40, page_size=32,
                             seqlens=(33, 1200, 64), sm_scale=S, seed=20), None),
    "sparse_h128": (Spec("sparse_h128", batch=2, q_len=1, num_heads=128, page_size=64,
                         seqlens=(5000, 3), topk=300, sm_scale=S, seed=16), None),
    "sparse_h16_lens": (Spec("sparse_h16_lens", batch=2, q_len=2, num_heads=16, page_size=16,
                             seqlens=(400, 90), topk=128, sm_scale=S, seed=17),
                        np.array([100, 0, 128, 64])),
    # fp8 rows (e4m3 values, one ue8m0 scale per 64, bf16 RoPE tail)
    "fp8_h128_edges": (Spec("fp8_h128_edges", batch=6, q_len=1, num_heads=128, page_size=64,
                            kv_format="fp8", seqlens=(1, 63, 64, 65, 700, 2001), sm_scale=S,
                            seed=31), None),
    "fp8_h16_page16": (Spec("fp8_h16_page16", batch=7, q_len=1, num_heads=16, page_size=16,
                            kv_format="fp8", seqlens=(0, 1, 15, 130, 511, 1000, 64), sm_scale=S,
                            scale_exp_range=(-6, 6), seed=32), None),
    "fp8_d512_verify": (Spec("fp8_d512_verify", batch=4, q_len=4, num_heads=16, d_qk=512,
                             kv_format="fp8", page_size=64, seqlens=(3, 131, 1000, 4),
                             causal=True, window=128, sink=True, sm_scale=1 / math.sqrt(512),
                             seed=33), None),
    "fp8_d512_h64": (Spec("fp8_d512_h64", batch=3, q_len=2, num_heads=64, d_qk=512,
                          kv_format="fp8", page_size=64, seqlens=(77, 700, 129), causal=True,
                          sm_scale=1 / math.sqrt(512), seed=34), None),
    "fp8_sparse_h128": (Spec("fp8_sparse_h128", batch=2, q_len=1, num_heads=128, page_size=64,
                             kv_format="fp8", seqlens=(5000, 3), topk=300, sm_scale=S, seed=35),
                        None),
    # 128 stacked rows with a causal window and a sink: the 128-row tile (fp8 ring conversion /
    # bf16 slots) when planned on one CU, 64-row tiles when planned on the device (short windows)
    "fp8_d512_h64_win_sink": (Spec("fp8_d512_h64_win_sink", batch=3, q_len=2, num_heads=64, d_qk=512,
                                   kv_format="fp8", page_size=64, seqlens=(77, 700, 129), causal=True,
                                   window=128, sink=True, sm_scale=1 / math.sqrt(512), seed=38), None),
    "h64_sq2_win_sink": (Spec("h64_sq2_win_sink", batch=3, q_len=2, num_heads=64, page_size=64,
                              seqlens=(5, 900, 200), causal=True, window=160, sink=True, sm_scale=S,
                              seed=39), None),
    # a sink with empty contexts: O = 0 and LSE = the sink logit for those requests
    "sink_empty": (Spec("sink_empty", batch=4, q_len=1, num_heads=16, page_size=16,
                        seqlens=(0, 5, 0, 300), sink=True, sm_scale=S, seed=36), None),
    "fp8_h128_sink_empty": (Spec("fp8_h128_sink_empty", batch=3, q_len=1, num_heads=128,
                                 page_size=64, kv_format="fp8", seqlens=(0, 700, 0), sink=True,
                                 sm_scale=S, seed=37), None),
    # index lists / windows of 16+ blocks over a few groups: each group split 16-17 ways when
    # planned on the device or on 1024 CUs (the combine's multi-batch merge, uneven last batch)
    "sparse_wide_h16": (Spec("sparse_wide_h16", batch=2, q_len=1, num_heads=16, page_size=64,
                             seqlens=(5000, 3000), topk=1024, sm_scale=S, seed=40), None),
    "win_wide_sink": (Spec("win_wide_sink", batch=2, q_len=2, num_heads=16, page_size=64,
                           seqlens=(3000, 1500), causal=True, window=1024, sink=True, sm_scale=S,
                           seed=41), None),
}


def _make(name):
    spec, tl = CASES[name]
    wl = make(spec, topk_lens=tl)
    if wl.indices is not None:
        # invalid entries: negative and past the sequence end are skipped
        idx = wl.indices.numpy()
        idx[0, 0, ::7] = -1
        idx[0, 0, 3::11] = int(wl.seqlens[0]) + 5
        wl.indices = torch.from_numpy(idx)
    return wl


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("cus", ["device", "one", "many"])
def test_parity(name, cus):
    wl = _make(name)
    num_cus = {"device": None, "one": 1, "many": 1024}[cus]
    print(f"[gpu] parity {name} cus={cus}", flush=True)
    out, lse, plan, used = H.run_gpu(wl, num_cus)
    O, L, A = H.oracle_of(wl, abs_mass=True)
    m = H.metrics(out, lse, O, L, A)
    print(f"[gpu]   {m}", flush=True)
    H.assert_parity(m, ctx=f"{name}/{cus}", scaled=H.scaled_bound(wl))
    want = H.plan_words(wl, used)
    got = plan.view(torch.int32).numpy()[:len(want)]
    assert np.array_equal(got, want), f"plan differs for {name}/{cus}"
    H.check_split_descriptors(plan, want, wl)


def test_page_permutation_bitwise():
    spec = dataclasses.replace(CASES["h128_edges"][0], page_seed=1)
    a = make(spec)
    b = make(dataclasses.replace(spec, page_seed=2))
    assert not torch.equal(a.block_table, b.block_table)
    print("[gpu] page permutation", flush=True)
    oa, la, _, _ = H.run_gpu(a)
    ob, lb, _, _ = H.run_gpu(b)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(la, lb)


def test_repeat_bitwise():
    wl = _make("h16_page16")
    print("[gpu] repeat", flush=True)
    o1, l1, _, _ = H.run_gpu(wl)
    o2, l2, _, _ = H.run_gpu(wl)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_uniform_scores_exact_mean():
    """q = 0 gives O = mean of the visible V rows and LSE = ln(count) exactly (closed form)."""
    spec = Spec("zero_q", batch=3, q_len=1, num_heads=16, page_size=16, seqlens=(1, 37, 256),
                sm_scale=S, seed=21)
    wl = make(spec)
    wl.q = torch.zeros_like(wl.q)
    out, lse, _, _ = H.run_gpu(wl)
    for b in range(3):
        L = int(wl.seqlens[b])
        mean = wl.request_rows(b).to(torch.float64)[:, :512].mean(dim=0)
        np.testing.assert_allclose(out[b, 0].to(torch.float64).numpy(),
                                   np.broadcast_to(mean.numpy(), (16, 512)), atol=2e-2, rtol=1e-2)
        np.testing.assert_allclose(lse[b, :, 0].numpy(), math.log(L), atol=1e-4)


def test_fp8_extreme_scales_uniform_scores():
    """q = 0 over fp8 rows whose scale exponents span [-100, 100]: O is the mean of the dequantised
    V rows (every exponent decoded exactly) and LSE = ln(count)."""
    spec = Spec("fp8_wide_scales", batch=2, q_len=1, num_heads=16, page_size=64, kv_format="fp8",
                seqlens=(70, 300), scale_exp_range=(-100, 100), sm_scale=S, seed=23)
    wl = make(spec)
    wl.q = torch.zeros_like(wl.q)
    print("[gpu] fp8 extreme scales", flush=True)
    out, lse, _, _ = H.run_gpu(wl)
    O, L, A = H.oracle_of(wl, abs_mass=True)
    m = H.metrics(out, lse, O, L, A)
    print(f"[gpu]   {m}", flush=True)
    H.assert_parity(m, ctx="fp8 extreme scales", scaled=H.scaled_bound(wl))
    for b in range(2):
        np.testing.assert_allclose(lse[b, :, 0].numpy(), math.log(int(wl.seqlens[b])), atol=1e-4)


def test_sparse_arange_equals_dense():
    spec = Spec("sp_eq", batch=2, q_len=1, num_heads=128, page_size=64, seqlens=(300, 64),
                sm_scale=S, seed=22)
    dense = make(spec)
    sp = make(dataclasses.replace(spec, topk=300))
    idx = np.full((2, 1, 300), -1, dtype=np.int32)
    idx[0, 0, :] = np.arange(300)
    idx[1, 0, :64] = np.arange(64)
    sp.indices = torch.from_numpy(idx)
    od, ld, _, _ = H.run_gpu(dense)
    os_, ls, _, _ = H.run_gpu(sp)
    m = H.metrics(os_, ls, od.to(torch.float64).numpy(), ld.to(torch.float64).numpy())
    assert m["max_abs"] <= 1e-2 and m["lse_max_abs"] <= 1e-4, m


FULL_SIZE = {2: CONFIGS[2], 3: CONFIGS[3], 4: CONFIGS[4], 5: CONFIGS[5],
             "s1": SUPPLEMENTARY["s1"], "s4": SUPPLEMENTARY["s4"],
             # config 3 with every scale exponent 0: held to the plain max-abs bound
             "3_exp0": dataclasses.replace(CONFIGS[3], name="dsv3_fp8_exp0", scale_exp_range=(0, 0))}


@pytest.mark.parametrize("cfg", list(FULL_SIZE))
def test_full_size_configs(cfg):
    """The benchmark workloads at their full sizes, in the launch configuration the bench uses."""
    wl = make(FULL_SIZE[cfg])
    print(f"[gpu] full-size config {cfg}", flush=True)
    out, lse, plan, used = H.run_gpu(wl)
    O, L, A = H.oracle_of(wl, abs_mass=True)
    m = H.metrics(out, lse, O, L, A)
    print(f"[gpu]   config {cfg}: max_abs={m['max_abs']:.4e} max_abs_scaled={m['max_abs_scaled']:.4e} "
          f"rel_l2={m['rel_l2']:.4e} lse={m['lse_max_abs']:.3e} (bound: "
          f"{'scaled' if H.scaled_bound(wl) else 'plain'})", flush=True)
    H.assert_parity(m, ctx=f"config {cfg}", scaled=H.scaled_bound(wl))
    want = H.plan_words(wl, used)
    assert np.array_equal(plan.view(torch.int32).numpy()[:len(want)], want)
    H.check_split_descriptors(plan, want, wl)


def test_graph_replay_matches_eager():
    """decode + combine captured in a HIP graph: every replay equals the eager result bitwise.

    Between replays the program does eager work of its own (the outputs are overwritten and the
    device synchronised), so a replay that depended on state left by the capture would show."""
    import mla_paged_latent_plan_amd as mla
    wl = _make("fp8_h128_edges")  # multi-split groups: decode partials, then the combine merge
    dev = H.to_device(wl)
    p = H.problem_of(wl, mla)
    runner = mla.MLADecode(p)
    s = wl.spec
    out = torch.empty(s.batch, s.q_len, s.num_heads, s.d_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(s.batch, s.num_heads, s.q_len, dtype=torch.float32, device="cuda")
    runner.plan_(dev.seqlens, dev.topk_lens)
    print("[gpu] graph replay: eager", flush=True)
    runner.decode_(dev.q, dev.cache, dev.block_table, dev.seqlens, s.sm_scale, out, lse,
                   indices=dev.indices, sink=dev.sink)
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        runner.decode_(dev.q, dev.cache, dev.block_table, dev.seqlens, s.sm_scale, out, lse,
                       indices=dev.indices, sink=dev.sink, stream=cap)
    torch.cuda.synchronize()
    for k in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        print(f"[gpu] graph replay {k}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {k}: out"
        assert torch.equal(lse, l_ref), f"replay {k}: lse"


@pytest.mark.parametrize("case", ["max_groups", "max_page", "h32_tiles"])
def test_maximum_sizes(case):
    """Limits of the library: the plan's 8192 query groups (per-group state held in LDS), pages of
    4096 rows (the largest accepted), and the 32-row tile (17..32 stacked rows) that no benchmark
    workload uses."""
    if case == "max_groups":
        rng = np.random.default_rng(71)
        lens = rng.integers(0, 40, 8192).astype(np.int32)  # empty requests included
        spec = Spec("max_groups", batch=8192, q_len=1, num_heads=16, page_size=16,
                    seqlens=tuple(int(x) for x in lens), sm_scale=S, seed=71)
    elif case == "max_page":
        spec = Spec("max_page", batch=2, q_len=1, num_heads=128, page_size=4096,
                    seqlens=(5000, 4096), sm_scale=S, seed=72)
    else:
        spec = Spec("h32_tiles", batch=5, q_len=2, num_heads=16, page_size=64,
                    seqlens=(2, 65, 700, 1999, 64), causal=True, sm_scale=S, seed=73)
    wl = make(spec)
    print(f"[gpu] maximum sizes: {case}", flush=True)
    out, lse, plan, used = H.run_gpu(wl)
    O, L, A = H.oracle_of(wl, abs_mass=True)
    m = H.metrics(out, lse, O, L, A)
    print(f"[gpu]   {m}", flush=True)
    H.assert_parity(m, ctx=case, scaled=H.scaled_bound(wl))
    want = H.plan_words(wl, used)
    assert np.array_equal(plan.view(torch.int32).numpy()[:len(want)], want)
    H.check_split_descriptors(plan, want, wl)


def test_sparse_duplicate_indices_count_per_occurrence():
    """Index lists with repeated entries: each occurrence is one more term of the softmax (the
    oracle's reading), so a list holding every index twice gives the same O as once and an LSE
    larger by ln 2."""
    spec = Spec("dup_idx", batch=2, q_len=1, num_heads=16, page_size=16, seqlens=(300, 90),
                topk=128, sm_scale=S, seed=38)
    wl = make(spec)
    idx = wl.indices.numpy().copy()
    idx[:, :, 64:] = idx[:, :, :64]  # entries 64..127 repeat entries 0..63
    wl.indices = torch.from_numpy(idx)
    print("[gpu] duplicate indices", flush=True)
    out, lse, _, _ = H.run_gpu(wl)
    O, L, A = H.oracle_of(wl, abs_mass=True)
    m = H.metrics(out, lse, O, L, A)
    print(f"[gpu]   {m}", flush=True)
    H.assert_parity(m, ctx="duplicate indices", scaled=H.scaled_bound(wl))
    half = dataclasses.replace(spec, topk=64, name="dup_idx_half")
    wl2 = make(half)
    wl2.indices = torch.from_numpy(np.ascontiguousarray(idx[:, :, :64]))
    out2, lse2, _, _ = H.run_gpu(wl2)
    np.testing.assert_allclose(lse.numpy(), lse2.numpy() + math.log(2.0), atol=1e-4)
    np.testing.assert_allclose(out.to(torch.float64).numpy(), out2.to(torch.float64).numpy(),
                               atol=2e-2)


@pytest.mark.parametrize("case", ["h16_bf16", "h128_fp8"])
def test_combine_past_64_splits(case):
    """One long request spread over the device's CUs: its group has more than 64 splits, so the
    combine walks its split LSEs and partial rows in several 64-split chunks."""
    if case == "h16_bf16":
        spec = Spec("long_h16", batch=2, q_len=1, num_heads=16, page_size=64,
                    seqlens=(131072, 100), sm_scale=S, seed=81)
    else:
        spec = Spec("long_h128_fp8", batch=2, q_len=1, num_heads=128, page_size=64,
                    kv_format="fp8", seqlens=(131072, 100), sm_scale=S, seed=82)
    wl = make(spec)
    print(f"[gpu] combine past 64 splits: {case}", flush=True)
    out, lse, plan, used = H.run_gpu(wl)
    want = H.plan_words(wl, used)
    words = plan.view(torch.int32).numpy()[:len(want)]
    assert np.array_equal(words, want)
    grp_ptr = words[16:16 + spec.batch + 1]
    nsplit = np.diff(grp_ptr)
    print(f"[gpu]   splits per group {nsplit.tolist()} on {used} CUs", flush=True)
    assert nsplit[0] > 64, f"the long request has only {nsplit[0]} splits"
    O, L, A = H.oracle_of(wl, abs_mass=True)
    m = H.metrics(out, lse, O, L, A)
    print(f"[gpu]   {m}", flush=True)
    H.assert_parity(m, ctx=case, scaled=H.scaled_bound(wl))


def test_plan_of_other_cu_count_gives_nan():
    """A plan built for another CU count (other units, other split records) is not used: the
    decode skips its work and the combine writes NaN to every output row and LSE."""
    import mla_paged_latent_plan_amd as mla
    wl = _make("h128_edges")
    dev = H.to_device(wl)
    p = H.problem_of(wl, mla)
    s = wl.spec
    cus = mla.device_num_cus()
    plan_bytes, part_bytes = mla.workspace_size(p, cus)
    plan_small, _ = mla.workspace_size(p, 1)
    plan = torch.zeros(max(plan_bytes, plan_small), dtype=torch.uint8, device="cuda")
    partials = torch.zeros(part_bytes, dtype=torch.uint8, device="cuda")
    out = torch.zeros(s.batch, s.q_len, s.num_heads, s.d_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(s.batch, s.num_heads, s.q_len, dtype=torch.float32, device="cuda")
    print("[gpu] plan of another CU count", flush=True)
    mla.mla_decode_plan(p, 1, dev.seqlens, None, plan)  # planned for one CU
    mla.mla_decode(p, cus, dev.q, dev.cache, dev.block_table, dev.seqlens, s.sm_scale, None, None,
                   plan, partials, out, lse)
    mla.mla_combine(p, cus, plan, partials, None, out, lse)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()
