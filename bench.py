"""Benchmark of MLA decode over a paged latent cache on one MI355X.

One step = mla_decode + mla_combine over one batch of the workload (the plan is built once per
forward and timed separately). Inputs are seeded synthetic tensors already resident in HBM.
Each timed step is preceded (outside its events) by a read-only sweep over a 1 GiB buffer that
was written once at set-up: it evicts the KV cache's lines from the 256 MB Infinity Cache and
leaves only clean lines there, so the decode reads the KV cache from HBM without also paying for
the write-back of an evicting kernel's dirty lines (a write fill of the same size is kept as an
option, --flush write). The step time (ms_per_step, value) brackets decode + combine with one pair
of events; a second loop with an event between the two kernels gives the per-kernel split
(decode_ms, combine_ms) and the decode time the roofline uses — that middle event record delays the
combine's dispatch, so the split sums to more than the step. Warm back-to-back figures are reported
separately, eager and as a replayed HIP graph of the same steps. The default run then times the
other workloads (configs 3, 4, 5, s1, s4: median decode, combine and step µs, each against its own
roofline) into a `per_config` object; their values are drawn on the GPU (workloads.make_on_device),
since drawing s4's 1.3 GB cache on the host takes about a minute. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|1|3|4|5|s1|s4] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "MLA decode: query tokens/s, achieved HBM TB/s & MFMA TFLOP/s, % of roofline"
DECODE_SRC = os.path.join(ROOT, "mla_paged_latent_plan_amd", "csrc", "decode.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    help="workload: 2 (default for decode), 1, 3 (default for kv_write), 4, 5, s1, s4")
    ap.add_argument("--op", choices=("decode", "kv_write", "absorb", "swa_runs", "gather",
                                     "sparse_prefill"), default="decode",
                    help="decode: mla_decode + mla_combine (the default); kv_write: mla_kv_write "
                         "of every row of the workload's requests in one launch; absorb: "
                         "mla_q_absorb + mla_v_up for --tokens query tokens (DeepSeek-V3 dims)")
    ap.add_argument("--tokens", type=int, default=64,
                    help="absorb: query tokens (64 = the dsv3 decode batch); swa_runs: tokens "
                         "(default 640)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other workloads' decode timings (per_config)")
    ap.add_argument("--flush", choices=("read", "write"), default="read",
                    help="cache eviction before each timed step: read-only 1 GiB sweep (default) "
                         "or a 512 MB fill that leaves dirty lines in the Infinity Cache")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    return ap.parse_args()


def emit(res):
    """Print the JSON line; with a CPU baseline in the same unit, also the GPU/CPU speed ratio."""
    cb = res.get("cpu_baseline")
    if cb and cb.get("value") and cb.get("unit") == res.get("unit"):
        res["gpu_cpu_speed_ratio"] = round(res["value"] / cb["value"], 1)
    print(json.dumps(res), flush=True)


def get_spec(name):
    from workloads import CONFIGS, SUPPLEMENTARY
    if name in SUPPLEMENTARY:
        return SUPPLEMENTARY[name]
    return CONFIGS[int(name)]


def algorithmic(wl):
    """Algorithmic HBM bytes and MFMA flops of one decode launch (rows each query may see)."""
    s = wl.spec
    from workloads.gen import cache_layout
    row_bytes = cache_layout(s.kv_format, s.d_qk, s.d_rope, s.page_size)["row_bytes"]
    if s.kv_format == "fp8":
        row_bytes += 8  # scale slot
    L = np.maximum(wl.seqlens.astype(np.int64), 0)
    Sq, H, B = s.q_len, s.num_heads, s.batch
    kv_rows = 0
    vis = 0
    pages = 0
    idx_bytes = 0
    for b in range(B):
        Lb = int(L[b])
        if s.topk > 0:
            idx = wl.indices[b].cpu().numpy()
            rows_b = set()
            for t in range(Sq):
                ok = idx[t][(idx[t] >= 0) & (idx[t] < Lb)]
                vis += len(ok)
                rows_b.update(ok.tolist())
            kv_rows += len(rows_b)
            pages += len({r // s.page_size for r in rows_b})
            idx_bytes += 4 * Sq * s.topk
        else:
            lo_union, n_b = Lb, 0
            for t in range(Sq):
                pos = Lb - Sq + t
                hi = min(Lb - 1, pos) if s.causal else Lb - 1
                lo = max(0, pos - s.window + 1) if s.window > 0 else 0
                if hi >= lo:
                    vis += hi - lo + 1
                    lo_union = min(lo_union, lo)
            n_b = Lb - lo_union if Lb > 0 else 0
            kv_rows += n_b
            if n_b:
                pages += (Lb - 1) // s.page_size - lo_union // s.page_size + 1
    q_bytes = B * Sq * H * s.d_qk * 2
    o_bytes = B * Sq * H * s.d_v * 2
    lse_bytes = B * Sq * H * 4
    total = kv_rows * row_bytes + q_bytes + o_bytes + lse_bytes + 4 * pages + idx_bytes
    flops = 2.0 * vis * H * (s.d_qk + s.d_v)
    return dict(bytes=int(total), kv_bytes=int(kv_rows * row_bytes), flops=flops,
                kv_rows=int(kv_rows), visible_pairs=int(vis))


# Sources whose change invalidates a kernel's committed HBM counter readings: the kernel itself,
# the shared argument/plan layout and, for decode, the plan (it decides the splits and partials).
KERNEL_SOURCES = {
    "decode": ("decode.hip", "plan.hip", "mla_internal.h"),
    "kvwrite": ("kvwrite.hip", "mla_internal.h"),
    "sparse_prefill": ("decode.hip", "plan.hip", "mla_internal.h"),
}


def source_hash(kernel="decode"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(os.path.dirname(DECODE_SRC), f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name, kernel="decode", what="hbm"):
    """HBM bytes (what="hbm") or L2 fetch bytes (what="l2_fetch") per launch of the kernel from the
    committed counter summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a plain copy's readings),
    if the kernel sources are unchanged since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_{what}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    key = f"{what}_bytes_per_launch"
    with open(path) as f:
        for line in f:
            m = re.match(r"- (source_hash|\w+_bytes_per_launch): (\S+)", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("source_hash") != source_hash(kernel) or key not in fields:
        return None
    return int(fields[key])


def cpu_baseline(wl, target_s):
    """The oracle, as it stands, on the first requests of the same workload."""
    import torch
    from oracle import attention as oatt
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    s = wl.spec

    def run(reqs):
        q = wl.q[reqs].to(torch.float64).numpy()
        seq = wl.seqlens[reqs]
        if s.topk > 0:
            idx = wl.indices[reqs].numpy()

            class Rows:  # rows are decoded when the oracle indexes them
                def __init__(self, b):
                    self.off = int(wl.row_offsets[b])

                def __getitem__(self, J):
                    J = torch.from_numpy(np.asarray(J, dtype=np.int64) + self.off)
                    return wl.rows_bf16[J].to(torch.float64).numpy()
            return oatt.mla_decode(q, lambda i: Rows(reqs[i]), seq, s.sm_scale, s.d_v,
                                   indices=idx)

        def rows(i):
            r = wl.request_rows(reqs[i])
            if s.kv_format == "bf16":
                return r.to(torch.float64).numpy()
            from oracle import fp8 as ofp8
            nope, sc, rope = r
            return ofp8.dequant_rows(nope.numpy(), sc.numpy(), rope.to(torch.float64).numpy())
        sink = None if wl.sink is None else wl.sink.to(torch.float64).numpy()
        return oatt.mla_decode(q, rows, seq, s.sm_scale, s.d_v, s.causal, s.window, sink=sink)

    t0 = time.perf_counter()
    run([0])
    t1 = time.perf_counter() - t0
    n = int(max(1, min(s.batch, target_s / max(t1, 1e-3))))
    reqs = list(range(n))
    # whole passes over the sample until the time target is reached (at most 10 passes)
    t0 = time.perf_counter()
    passes = 0
    while True:
        run(reqs)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or passes >= 10:
            break
    return dict(value=passes * n * s.q_len / dt, unit="query tokens/s", cores=int(threads),
                kind="oracle",
                sample=f"{passes} pass(es) over the first {n} of {s.batch} requests of the same "
                       f"workload, float64 numpy oracle, {dt:.1f} s",
                os_cpu_count=os.cpu_count(), affinity=len(os.sched_getaffinity(0)),
                cpu_model=cpu_model())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_kv_write(kv_c, k_pe, fmt, target_s):
    """The cache-write oracle, as it stands, on the first rows of the same inputs."""
    from oracle import kvwrite
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < target_s and n < kv_c.shape[0]:
        kvwrite.encode_row(kv_c[n], k_pe[n], fmt)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=round(n / dt, 1), unit="rows/s", cores=1, kind="oracle",
                sample=f"the first {n} rows of the same inputs, float64 numpy/python oracle "
                       f"(oracle/kvwrite.py encode_row), one thread, {dt:.1f} s")


def bench_kv_write(args):
    """mla_kv_write of every row of the workload's requests (in request order through the block
    table) in one launch: the cache write a prefill of these contexts would do."""
    import torch
    import mla_paged_latent_plan_amd as mla
    from workloads import make
    from workloads.gen import cache_layout

    s = get_spec(args.config or "3")
    wl = make(s)
    dev = torch.device("cuda:0")
    lay = cache_layout(s.kv_format, s.d_qk, s.d_rope, s.page_size)
    bt = wl.block_table.numpy()
    L = np.maximum(wl.seqlens.astype(np.int64), 0)
    req = np.repeat(np.arange(s.batch), L)
    pos = np.concatenate([np.arange(x) for x in L])
    slots = bt[req, pos // s.page_size].astype(np.int64) * s.page_size + pos % s.page_size
    n = len(slots)
    g = torch.Generator().manual_seed(s.seed + 500)
    kv_c_h = torch.randn(n, s.d_qk - s.d_rope, generator=g).to(torch.bfloat16)
    k_pe_h = torch.randn(n, s.d_rope, generator=g).to(torch.bfloat16)
    p = mla.make_problem(s.batch, s.q_len, s.num_heads, s.d_qk,
                         mla.MLA_KV_BF16 if s.kv_format == "bf16" else mla.MLA_KV_FP8,
                         s.page_size, wl.page_stride, wl.num_pages, int(bt.shape[1]))
    kv_c, k_pe = kv_c_h.to(dev), k_pe_h.to(dev)
    slot_d = torch.from_numpy(slots).to(dev)
    cache = wl.cache.to(dev)
    stream = torch.cuda.current_stream()
    sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sweep_out = torch.empty(1, dtype=torch.float32, device=dev)
    write = lambda: mla.mla_kv_write(p, kv_c, k_pe, slot_d, cache, stream)
    for _ in range(args.warmup):
        write()
    torch.cuda.synchronize()
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev()) for _ in range(K)]
    for k in range(K):
        if not args.no_flush:
            torch.sum(sweep, dim=0, out=sweep_out[0])
        a, b = evs[k]
        a.record(stream)
        write()
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    # context: a plain device-to-device copy of the rows' input bytes (read + write) after the
    # same eviction, the rate a pure streaming kernel reaches on this GPU
    src = torch.empty(n * 2 * s.d_qk, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cms = []
    for _ in range(5):
        torch.sum(sweep, dim=0, out=sweep_out[0])
        a, b = ev(), ev()
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        cms.append(a.elapsed_time(b))
    copy_gbs = 2 * src.numel() / (float(np.median(cms)) / 1e3) / 1e9
    del src, dst
    out_row = lay["row_bytes"] + (8 if s.kv_format == "fp8" else 0)
    alg_bytes = n * (2 * s.d_qk + out_row + 8)
    t = float(ms.mean()) / 1e3
    gbs = alg_bytes / t / 1e9
    res = {
        "metric": "MLA cache write: rows/s, achieved HBM GB/s, % of roofline",
        "value": round(n / t, 1), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->" + ("bf16" if s.kv_format == "bf16" else "fp8-e4m3/ue8m0"),
        "data": "synthetic",
        "config": {"workload": f"kv_write {s.name}: {n} rows of d_qk {s.d_qk} written into pages of "
                               f"{s.page_size} ({s.kv_format} rows of {lay['row_bytes']} B)",
                   "rows": n, "parallelism": "single-gpu"},
        "roofline": dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4),
                         traffic=measured_traffic(s.name, "kvwrite")),
        "ms_p10_p90": [round(float(np.percentile(ms, 10)), 4),
                       round(float(np.percentile(ms, 90)), 4)],
        "algorithmic_bytes": int(alg_bytes),
        "device_copy_gbs": round(copy_gbs, 1),
        "cache_eviction": "none" if args.no_flush else "read-only 1 GiB sweep",
        "source_hash": source_hash("kvwrite"),
    }
    if not args.no_cpu:
        m = min(n, 20000)  # the oracle is timed on a bounded prefix of the rows
        res["cpu_baseline"] = cpu_kv_write(kv_c_h[:m].to(torch.float64).numpy(),
                                           k_pe_h[:m].to(torch.float64).numpy(), s.kv_format,
                                           args.cpu_seconds)
    emit(res)


def bench_absorb(args):
    """mla_q_absorb then mla_v_up for T query tokens of DeepSeek-V3 shape (128 heads, P 128,
    L 512, R 64, V 128): the per-head GEMMs on either side of the decode."""
    import torch
    import mla_paged_latent_plan_amd as mla
    T, Hh, P, L, R, V = args.tokens, 128, 128, 512, 64, 128
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(2000 + T)
    mk = lambda *sh, sc=1.0: (torch.randn(*sh, generator=g) * sc).to(torch.bfloat16).to(dev)
    q_nope, q_pe = mk(T, Hh, P), mk(T, Hh, R)
    w_uk, w_uv = mk(Hh, L, P, sc=P ** -0.5), mk(Hh, V, L, sc=L ** -0.5)
    o = mk(T, Hh, L)
    q_out = torch.empty(T, Hh, L + R, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, Hh, V, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sweep_out = torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        mla.mla_q_absorb(q_nope, q_pe, w_uk, q_out, stream)
        mla.mla_v_up(o, w_uv, out, stream)
    torch.cuda.synchronize()
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev(), ev()) for _ in range(K)]
    for k in range(K):
        if not args.no_flush:
            torch.sum(sweep, dim=0, out=sweep_out[0])
        a, m, e = evs[k]
        a.record(stream)
        mla.mla_q_absorb(q_nope, q_pe, w_uk, q_out, stream)
        m.record(stream)
        mla.mla_v_up(o, w_uv, out, stream)
        e.record(stream)
    torch.cuda.synchronize()
    qa = np.array([a.elapsed_time(m) for a, m, _ in evs])
    vu = np.array([m.elapsed_time(e) for _, m, e in evs])
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    qa_bytes = 2 * (T * Hh * P + T * Hh * R + Hh * L * P + T * Hh * (L + R))
    vu_bytes = 2 * (T * Hh * L + Hh * V * L + T * Hh * V)
    flops = 2.0 * T * Hh * L * (P + V)
    t = float((qa + vu).mean()) / 1e3
    gbs = (qa_bytes + vu_bytes) / t / 1e9
    bound = "hbm" if flops / (qa_bytes + vu_bytes) < MFMA_BF16_PEAK_TFS / HBM_PEAK_GBS * 1e3 else "mfma"
    roof = (dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                 frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None) if bound == "hbm" else
            dict(bound="mfma", achieved=round(flops / t / 1e12, 2), peak=MFMA_BF16_PEAK_TFS,
                 unit="TFLOP/s", frac=round(flops / t / 1e12 / MFMA_BF16_PEAK_TFS, 4), traffic=None))
    res = {
        "metric": "MLA absorption GEMMs: query tokens/s, achieved HBM GB/s, % of roofline",
        "value": round(T / t, 1), "unit": "query tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(float((qa + vu).mean()), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"absorb: {T} query tokens x {Hh} heads, W_UK [{Hh},{L},{P}], "
                               f"W_UV [{Hh},{V},{L}], RoPE {R}", "tokens": T,
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "q_absorb_ms": round(float(qa.mean()), 4), "v_up_ms": round(float(vu.mean()), 4),
        "q_absorb_gbs": round(qa_bytes / (float(qa.mean()) / 1e3) / 1e9, 1),
        "v_up_gbs": round(vu_bytes / (float(vu.mean()) / 1e3) / 1e9, 1),
        "algorithmic_bytes": int(qa_bytes + vu_bytes), "algorithmic_flops": flops,
        "cache_eviction": "none" if args.no_flush else "read-only 1 GiB sweep",
    }
    if not args.no_cpu:
        from oracle import absorb
        t0 = time.perf_counter()
        n = 0
        qn = q_nope.cpu().to(torch.float64).numpy()
        wk = w_uk.cpu().to(torch.float64).numpy()
        oo = o.cpu().to(torch.float64).numpy()
        wv = w_uv.cpu().to(torch.float64).numpy()
        while time.perf_counter() - t0 < args.cpu_seconds:
            absorb.q_absorb(qn, wk)
            absorb.v_up(oo, wv)
            n += 1
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = os.cpu_count() or 1
        res["cpu_baseline"] = dict(value=round(n * T / dt, 1), unit="query tokens/s",
                                   cores=threads, kind="oracle",
                                   sample=f"{n} pass(es) over all {T} tokens, float64 numpy oracle "
                                          f"(oracle/absorb.py), {dt:.1f} s")
    emit(res)


def bench_sparse_prefill(args):
    """mla_sparse_prefill (metadata fill, plan, decode with per-row maxima, combine) on the
    DeepSeek-V3.2-shaped prefill: 4096 tokens x 128 heads, 576-wide rows, top-k 2048 of a
    32768-row buffer. One step = one call; the decode kernel takes nearly all of it."""
    import torch
    import mla_paged_latent_plan_amd as mla
    from workloads import gen
    spec = gen.SPARSE_PREFILL["dsv32_prefill"]
    dev = torch.device("cuda:0")
    q, kv, idx = gen.make_sparse_prefill(spec)
    valid = int(((idx >= 0) & (idx < spec.s_kv)).sum())
    qd, kvd, idd = q.to(dev), kv.to(dev), idx.to(dev)
    cus = mla.device_num_cus()
    H, s_q = spec.num_heads, spec.s_q
    ws = torch.empty(mla.sparse_prefill_workspace_size(s_q, H, spec.d_qk, spec.topk, spec.s_kv, cus),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(s_q, H, 512, dtype=torch.bfloat16, device=dev)
    mlog = torch.empty(H, s_q, device=dev)
    lse = torch.empty(H, s_q, device=dev)
    stream = torch.cuda.current_stream()
    sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sweep_out = torch.empty(1, dtype=torch.float32, device=dev)
    call = lambda: mla.mla_sparse_prefill(qd, kvd, idd, spec.sm_scale, ws, out, mlog, lse, cus,
                                          stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev()) for _ in range(K)]
    for k in range(K):
        if not args.no_flush:
            torch.sum(sweep, dim=0, out=sweep_out[0])
        a, e = evs[k]
        a.record(stream)
        call()
        e.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(e) for a, e in evs])
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    t = float(ms.mean()) / 1e3
    flops = 2.0 * valid * H * (spec.d_qk + 512)
    nbytes = 2 * (q.numel() + kv.numel() + out.numel()) + 4 * (idx.numel() + 2 * H * s_q)
    res = {
        "metric": "MLA sparse prefill: query tokens/s, achieved MFMA TFLOP/s, % of roofline",
        "value": round(s_q / t, 1), "unit": "query tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"sparse prefill {spec.name}: {s_q} tokens x {H} heads, d_qk "
                               f"{spec.d_qk}, d_v 512, top-k {spec.topk} of {spec.s_kv} rows",
                   "tokens": s_q, "parallelism": "single-gpu"},
        "roofline": dict(bound="mfma", achieved=round(flops / t / 1e12, 2),
                         peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s",
                         frac=round(flops / t / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                         traffic=None,
                         kernel="the whole call (metadata fill, plan, decode, combine)"),
        # FETCH_SIZE + WRITE_SIZE of the decode kernel: L2 misses, mostly served by the Infinity
        # Cache (the rows are gathered many times over), so not an HBM figure
        "l2_fetch_bytes": measured_traffic("dsv32", kernel="sparse_prefill", what="l2_fetch"),
        "ms_p10_p90": [round(float(np.percentile(ms, 10)), 4),
                       round(float(np.percentile(ms, 90)), 4)],
        "algorithmic_flops": flops, "algorithmic_bytes": int(nbytes), "valid_entries": valid,
        "cache_eviction": "none" if args.no_flush else "read-only 1 GiB sweep",
    }
    if not args.no_cpu:
        from oracle.sparse_prefill import sparse_prefill
        qn, kvn, ixn = q.float().numpy(), kv.float().numpy(), idx.numpy()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds and n < s_q:
            sparse_prefill(qn, kvn, ixn, spec.sm_scale, tokens=[n])
            n += 1
        dt = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = os.cpu_count() or 1
        res["cpu_baseline"] = dict(value=round(n / dt, 2), unit="query tokens/s", cores=threads,
                                   kind="oracle",
                                   sample=f"the first {n} of {s_q} tokens, float64 numpy oracle "
                                          f"(oracle/sparse_prefill.py), {dt:.1f} s")
    emit(res)


def bench_swa_runs(args):
    """mla_swa_runs over T tokens' 128-row windows (+ 3 drafts) in a ring of slots, pages of 64:
    the plan step of sliding-window layers, run once per forward."""
    import torch
    import mla_paged_latent_plan_amd as mla
    T = args.tokens if args.tokens != 64 else 640
    topk, page = 131, 64
    g = np.random.default_rng(3000 + T)
    base = g.integers(0, 1 << 20, T)
    kv = (base[:, None] + np.arange(topk)[None, :]).astype(np.int32)  # mostly one or two runs
    lengths = g.integers(1, topk + 1, T).astype(np.int32)
    dev = torch.device("cuda:0")
    kv_d, len_d = torch.from_numpy(kv).to(dev), torch.from_numpy(lengths).to(dev)
    runs = torch.empty(T, 4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        mla.mla_swa_runs(kv_d, len_d, page, 1, runs, stream)
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        mla.mla_swa_runs(kv_d, len_d, page, 1, runs, stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    nbytes = T * topk * 4 + T * 4 + T * 16
    t = float(ms.mean()) / 1e3
    res = {
        "metric": "MLA sliding-window run plan: tokens/s, achieved HBM GB/s",
        "value": round(T / t, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"swa_runs: {T} tokens x {topk}-slot windows, pages of {page}",
                   "tokens": T, "parallelism": "single-gpu"},
        "roofline": dict(bound="hbm", achieved=round(nbytes / t / 1e9, 1), peak=HBM_PEAK_GBS,
                         unit="GB/s", frac=round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), traffic=None),
        "note": "latency-bound: one launch over a few hundred KB",
    }
    if not args.no_cpu:
        from oracle import swa_runs
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            swa_runs.swa_runs(kv, lengths, page, 1)
            n += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=round(n * T / dt, 1), unit="tokens/s", cores=1,
                                   kind="oracle", sample=f"{n} pass(es) over all {T} tokens, "
                                                         f"pure-Python oracle, {dt:.1f} s")
    emit(res)


def bench_gather(args):
    """mla_gather_context of the whole context of every request of the workload in one launch (the
    rows a chunked-context prefill over these contexts gathers), fp8 rows widened to bf16."""
    import torch
    import mla_paged_latent_plan_amd as mla
    from workloads import make
    from workloads.gen import cache_layout

    s = get_spec(args.config or "3")
    wl = make(s)
    dev = torch.device("cuda:0")
    lay = cache_layout(s.kv_format, s.d_qk, s.d_rope, s.page_size)
    lens = np.maximum(wl.seqlens.astype(np.int64), 0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t2s = np.repeat(np.arange(s.batch), lens).astype(np.int32)
    n = int(cu[-1])
    p = mla.make_problem(s.batch, s.q_len, s.num_heads, s.d_qk,
                         mla.MLA_KV_BF16 if s.kv_format == "bf16" else mla.MLA_KV_FP8,
                         s.page_size, wl.page_stride, wl.num_pages, int(wl.block_table.shape[1]))
    bt, cu_d, t2s_d = wl.block_table.to(dev), torch.from_numpy(cu).to(dev), torch.from_numpy(t2s).to(dev)
    cache = wl.cache.to(dev)
    dst = torch.empty(n, s.d_qk, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sweep_out = torch.empty(1, dtype=torch.float32, device=dev)
    run = lambda: mla.mla_gather_context(p, bt, cu_d, None, t2s_d, cache, dst, stream)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for a, b in evs:
        if not args.no_flush:
            torch.sum(sweep, dim=0, out=sweep_out[0])
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    in_row = lay["row_bytes"] + (8 if s.kv_format == "fp8" else 0)
    nbytes = n * (in_row + 2 * s.d_qk + 4) + 4 * (s.batch + 1) + 4 * int(np.sum(-(-lens // s.page_size)))
    t = float(ms.mean()) / 1e3
    gbs = nbytes / t / 1e9
    res = {
        "metric": "MLA context gather: rows/s, achieved HBM GB/s, % of roofline",
        "value": round(n / t, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8-e4m3/ue8m0" if s.kv_format == "fp8" else "bf16") + "->bf16",
        "data": "synthetic",
        "config": {"workload": f"gather {s.name}: all {n} context rows of {s.batch} requests, "
                               f"pages of {s.page_size}", "rows": n, "parallelism": "single-gpu"},
        "roofline": dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None),
        "ms_p10_p90": [round(float(np.percentile(ms, 10)), 4), round(float(np.percentile(ms, 90)), 4)],
        "algorithmic_bytes": int(nbytes),
        "cache_eviction": "none" if args.no_flush else "read-only 1 GiB sweep",
    }
    if not args.no_cpu:
        from oracle import gather
        cache_h, bt_h = wl.cache.numpy(), wl.block_table.numpy()
        k, passes = min(n, 4000), 0
        t0 = time.perf_counter()
        while passes == 0 or time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            gather.gather_context(cache_h, bt_h, cu, None, t2s[:k], s.kv_format, s.d_qk, s.d_rope,
                                  s.page_size)  # output rows 0 .. k - 1 of the same gather
            passes += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=round(passes * k / dt, 1), unit="rows/s", cores=1,
                                   kind="oracle", sample=f"{passes} pass(es) over the first {k} "
                                   f"output rows, float64 numpy oracle (oracle/gather.py), {dt:.1f} s")
    emit(res)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.op == "kv_write":
        return bench_kv_write(args)
    if args.op == "absorb":
        return bench_absorb(args)
    if args.op == "swa_runs":
        return bench_swa_runs(args)
    if args.op == "sparse_prefill":
        return bench_sparse_prefill(args)
    if args.op == "gather":
        return bench_gather(args)
    import torch
    import mla_paged_latent_plan_amd as mla
    from workloads import make

    from mla_paged_latent_plan_amd import _lib
    build_id = _lib.check_build_id()
    spec = get_spec(args.config or "2")
    wl = make(spec)
    dev = torch.device("cuda:0")
    s = spec
    p = mla.make_problem(s.batch, s.q_len, s.num_heads, s.d_qk,
                         mla.MLA_KV_BF16 if s.kv_format == "bf16" else mla.MLA_KV_FP8,
                         s.page_size, wl.page_stride, wl.num_pages, int(wl.block_table.shape[1]),
                         s.topk, s.causal, s.window)
    num_cus = s.plan_cus or mla.device_num_cus()
    runner = mla.MLADecode(p, num_cus, device=dev)
    q = wl.q.to(dev)
    cache = wl.cache.to(dev)
    bt = wl.block_table.to(dev)
    seq = torch.from_numpy(wl.seqlens).to(dev)
    idx = None if wl.indices is None else wl.indices.to(dev)
    sink = None if wl.sink is None else wl.sink.to(dev)
    out = torch.empty(s.batch, s.q_len, s.num_heads, s.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(s.batch, s.num_heads, s.q_len, dtype=torch.float32, device=dev)
    if args.flush == "read":
        sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, written once
        sweep_out = torch.empty(1, dtype=torch.float32, device=dev)
        evict = lambda k: torch.sum(sweep, dim=0, out=sweep_out[0])
    else:
        fill = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        evict = lambda k: fill.fill_(k & 0xFF)
    stream = torch.cuda.current_stream()

    def plan():
        mla.mla_decode_plan(p, num_cus, seq, None if wl.topk_lens is None else
                            wl.topk_lens.to(dev), runner.plan, stream)

    def decode(st=None):
        mla.mla_decode(p, num_cus, q, cache, bt, seq, s.sm_scale, idx, sink, runner.plan,
                       runner.partials, out, lse, st or stream)

    def combine(st=None):
        mla.mla_combine(p, num_cus, runner.plan, runner.partials, sink, out, lse, st or stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    # plan (once per forward; timed on its own)
    plan()
    torch.cuda.synchronize()
    pe = [(ev(), ev()) for _ in range(10)]
    for a, b in pe:
        a.record(stream)
        plan()
        b.record(stream)
    torch.cuda.synchronize()
    plan_ms = float(np.median([a.elapsed_time(b) for a, b in pe]))

    for _ in range(args.warmup):
        decode()
        combine()
    torch.cuda.synchronize()

    K = args.steps
    evs = [(ev(), ev(), ev()) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        if not args.no_flush:
            evict(k)
        a, m, e = evs[k]
        a.record(stream)
        decode()
        m.record(stream)
        combine()
        e.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / K * 1e3
    dec_ms = np.array([a.elapsed_time(m) for a, m, _ in evs])
    com_ms = np.array([m.elapsed_time(e) for _, m, e in evs])
    # the step itself, timed without the marker between the two kernels (the loop above gives the
    # per-kernel split; its middle event record can delay the combine's dispatch)
    sevs = [(ev(), ev()) for _ in range(K)]
    for k in range(K):
        if not args.no_flush:
            evict(k)
        a, e = sevs[k]
        a.record(stream)
        decode()
        combine()
        e.record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(e) for a, e in sevs])

    # warm back-to-back (cache-resident) for context
    wa, wb = ev(), ev()
    wa.record(stream)
    for _ in range(K):
        decode()
        combine()
    wb.record(stream)
    torch.cuda.synchronize()
    warm_ms = wa.elapsed_time(wb) / K

    # the same K steps captured once in a HIP graph and replayed (warm cache, no launch gaps)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(K):
            decode(cap)
            combine(cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ga, gb = ev(), ev()
    ga.record(stream)
    graph.replay()
    gb.record(stream)
    torch.cuda.synchronize()
    graph_ms = ga.elapsed_time(gb) / K

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    alg = algorithmic(wl)
    dec_s = float(dec_ms.mean()) / 1e3
    ms = float(step_ms.mean())
    tokens = s.batch * s.q_len
    achieved_gbs = alg["bytes"] / dec_s / 1e9
    achieved_tfs = alg["flops"] / dec_s / 1e12
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "hbm" if alg["flops"] / alg["bytes"] < ridge else "mfma"
    traffic = measured_traffic(s.name)
    if bound == "hbm":
        roof = dict(bound="hbm", achieved=round(achieved_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved_gbs / HBM_PEAK_GBS, 4), traffic=traffic)
    else:
        roof = dict(bound="mfma", achieved=round(achieved_tfs, 2), peak=MFMA_BF16_PEAK_TFS,
                    unit="TFLOP/s", frac=round(achieved_tfs / MFMA_BF16_PEAK_TFS, 4),
                    traffic=traffic)
    res = {
        "metric": METRIC,
        "value": round(tokens / (ms / 1e3), 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.kv_format if s.kv_format == "bf16" else "fp8-e4m3/bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{s.name}: batch {s.batch}, q_len {s.q_len}, {s.num_heads} heads, "
                        f"d_qk {s.d_qk}/d_v {s.d_v} {s.kv_format} rows, page {s.page_size}, "
                        + (f"lengths U[{s.len_range[0]},{s.len_range[1]}]" if s.len_range
                           else f"lengths {list(s.seqlens)[:4]}")
                        + (f", causal" if s.causal else "") + (f", window {s.window}" if s.window else "")
                        + (f", sink" if s.sink else "") + (f", top-k {s.topk}" if s.topk else ""),
            "global_batch": s.batch, "seq_len": int(wl.seqlens.max()), "parallelism": "single-gpu",
            "num_cus_planned": num_cus,
        },
        "roofline": roof,
        "hbm_tbs": round(achieved_gbs / 1e3, 3),
        "hbm_frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "mfma_tflops": round(achieved_tfs, 2),
        "mfma_frac": round(achieved_tfs / MFMA_BF16_PEAK_TFS, 4),
        "ms_per_step_median": round(float(np.median(step_ms)), 4),
        "ms_per_step_p10_p90": [round(float(np.percentile(step_ms, 10)), 4),
                                round(float(np.percentile(step_ms, 90)), 4)],
        "decode_ms": round(float(dec_ms.mean()), 4),
        "decode_ms_median": round(float(np.median(dec_ms)), 4),
        "decode_ms_p10_p90": [round(float(np.percentile(dec_ms, 10)), 4),
                              round(float(np.percentile(dec_ms, 90)), 4)],
        "combine_ms": round(float(com_ms.mean()), 4),
        "decode_plus_combine_ms_with_marker": round(float((dec_ms + com_ms).mean()), 4),
        "plan_ms": round(plan_ms, 4),
        "warm_ms_per_step": round(warm_ms, 4),
        "graph_warm_ms_per_step": round(graph_ms, 4),
        "wall_ms_per_step_with_flush": round(wall, 4),
        "cache_eviction": "none" if args.no_flush else
                          ("read-only 1 GiB sweep" if args.flush == "read" else "512 MB write fill"),
        # the whole step (decode + combine) against the same roofline
        "step_hbm_frac": round(alg["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(alg["flops"] / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "algorithmic_bytes": alg["bytes"],
        "algorithmic_flops": alg["flops"],
        "source_hash": source_hash(),
        "build_id": build_id,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    if args.config is None and not args.no_per_config:
        del q, cache, bt, runner, graph
        torch.cuda.empty_cache()
        res["per_config"] = per_config(args, evict)
    emit(res)


PER_CONFIG = ("3", "4", "5", "s1", "s4")


def per_config(args, evict):
    """Decode and combine times of the other workloads (GPU only, values drawn on the device:
    workloads.make_on_device), each against its own roofline."""
    import torch
    import mla_paged_latent_plan_amd as mla
    from workloads import make_on_device

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out_all = {}
    K = max(5, min(args.steps, 20))
    for name in PER_CONFIG:
        s = get_spec(name)
        wl = make_on_device(s, dev)
        p = mla.make_problem(s.batch, s.q_len, s.num_heads, s.d_qk,
                             mla.MLA_KV_BF16 if s.kv_format == "bf16" else mla.MLA_KV_FP8,
                             s.page_size, wl.page_stride, wl.num_pages, int(wl.block_table.shape[1]),
                             s.topk, s.causal, s.window)
        num_cus = s.plan_cus or mla.device_num_cus()
        runner = mla.MLADecode(p, num_cus, device=dev)
        seq = torch.from_numpy(wl.seqlens).to(dev)
        out = torch.empty(s.batch, s.q_len, s.num_heads, s.d_v, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(s.batch, s.num_heads, s.q_len, dtype=torch.float32, device=dev)
        mla.mla_decode_plan(p, num_cus, seq, None, runner.plan, stream)

        def decode():
            mla.mla_decode(p, num_cus, wl.q, wl.cache, wl.block_table, seq, s.sm_scale, wl.indices,
                           wl.sink, runner.plan, runner.partials, out, lse, stream)

        def combine():
            mla.mla_combine(p, num_cus, runner.plan, runner.partials, wl.sink, out, lse, stream)

        for _ in range(3):
            decode()
            combine()
        torch.cuda.synchronize()
        ev = lambda: torch.cuda.Event(enable_timing=True)
        evs = [(ev(), ev(), ev()) for _ in range(K)]
        for k in range(K):
            if not args.no_flush:
                evict(k)
            a, m, e = evs[k]
            a.record(stream)
            decode()
            m.record(stream)
            combine()
            e.record(stream)
        torch.cuda.synchronize()
        sevs = [(ev(), ev()) for _ in range(K)]
        for k in range(K):
            if not args.no_flush:
                evict(k)
            a, e = sevs[k]
            a.record(stream)
            decode()
            combine()
            e.record(stream)
        torch.cuda.synchronize()
        dec = np.array([a.elapsed_time(m) for a, m, _ in evs]) * 1e3
        com = np.array([m.elapsed_time(e) for _, m, e in evs]) * 1e3
        step = np.array([a.elapsed_time(e) for a, e in sevs]) * 1e3
        alg = algorithmic(wl)
        ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
        bound = "hbm" if alg["flops"] / alg["bytes"] < ridge else "mfma"
        dec_s = float(np.median(dec)) / 1e6
        step_s = float(np.median(step)) / 1e6
        if bound == "hbm":
            frac = alg["bytes"] / dec_s / 1e9 / HBM_PEAK_GBS
            sfrac = alg["bytes"] / step_s / 1e9 / HBM_PEAK_GBS
        else:
            frac = alg["flops"] / dec_s / 1e12 / MFMA_BF16_PEAK_TFS
            sfrac = alg["flops"] / step_s / 1e12 / MFMA_BF16_PEAK_TFS
        out_all[name] = {
            "workload": s.name,
            "decode_us_median": round(float(np.median(dec)), 2),
            "combine_us_median": round(float(np.median(com)), 2),
            "step_us_median": round(float(np.median(step)), 2),
            "value": round(s.batch * s.q_len / step_s, 1),
            "unit": "query tokens/s",
            "bound": bound,
            "frac": round(frac, 4),
            "step_frac": round(sfrac, 4),
            "hbm_tbs": round(alg["bytes"] / dec_s / 1e12, 3),
            "mfma_tflops": round(alg["flops"] / dec_s / 1e12, 2),
            "algorithmic_bytes": alg["bytes"],
            "algorithmic_flops": alg["flops"],
            "splits": int(runner.plan[:16].view(torch.int32)[3].item()),  # plan header word 3: the split count
        }
        del wl, runner, out, lse, seq
        torch.cuda.empty_cache()
    return out_all


if __name__ == "__main__":
    main()
