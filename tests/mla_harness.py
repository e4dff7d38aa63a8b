"""Shared helpers of the GPU tests: move a workload to the device, run the HIP path through the
C ABI, evaluate the oracle on the same inputs and measure the difference."""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

from oracle import attention as oatt
from oracle import fp8 as ofp8
from oracle import plan as oplan

# Parity bar for the decode outputs (bf16 O against the float64 oracle).
REL_L2 = 5e-3
MAX_ABS = 2e-2
LSE_ABS = 1e-3


def problem_of(wl, mla):
    s = wl.spec
    return mla.make_problem(
        batch=s.batch, q_len=s.q_len, num_heads=s.num_heads, d_qk=s.d_qk,
        kv_format=mla.MLA_KV_BF16 if s.kv_format == "bf16" else mla.MLA_KV_FP8,
        page_size=s.page_size, page_stride_bytes=wl.page_stride, num_pages=wl.num_pages,
        max_pages_per_seq=int(wl.block_table.shape[1]), topk=s.topk, causal=s.causal,
        window=s.window, d_v=s.d_v, d_rope=s.d_rope)


@dataclasses.dataclass
class DeviceInputs:
    q: torch.Tensor
    cache: torch.Tensor
    block_table: torch.Tensor
    seqlens: torch.Tensor
    indices: Optional[torch.Tensor]
    topk_lens: Optional[torch.Tensor]
    sink: Optional[torch.Tensor]


def to_device(wl, device="cuda") -> DeviceInputs:
    return DeviceInputs(
        q=wl.q.to(device),
        cache=wl.cache.to(device),
        block_table=wl.block_table.to(device),
        seqlens=torch.from_numpy(wl.seqlens).to(device),
        indices=None if wl.indices is None else wl.indices.to(device),
        topk_lens=None if wl.topk_lens is None else wl.topk_lens.to(device),
        sink=None if wl.sink is None else wl.sink.to(device))


def run_gpu(wl, num_cus: Optional[int] = None, dev: Optional[DeviceInputs] = None):
    """plan + decode + combine through the C ABI; returns (out bf16, lse fp32, plan words) on CPU."""
    import mla_paged_latent_plan_amd as mla
    dev = dev or to_device(wl)
    p = problem_of(wl, mla)
    if num_cus is None:
        num_cus = wl.spec.plan_cus or mla.device_num_cus()
    runner = mla.MLADecode(p, num_cus)
    out, lse = runner(dev.q, dev.cache, dev.block_table, dev.seqlens, wl.spec.sm_scale,
                      indices=dev.indices, sink=dev.sink, topk_lens=dev.topk_lens)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), runner.plan.cpu(), num_cus


def dense_rows(wl, b: int) -> np.ndarray:
    """Oracle-side float64 rows of request b, decoded from the logical (unpaged) rows."""
    r = wl.request_rows(b)
    if wl.spec.kv_format == "bf16":
        return r.to(torch.float64).numpy()
    nope, scales, rope = r
    return ofp8.dequant_rows(nope.numpy(), scales.numpy(), rope.to(torch.float64).numpy())


def dense_rows_at(wl, b: int, J: np.ndarray) -> np.ndarray:
    """Oracle-side float64 rows J (request-local positions) of request b."""
    off = int(wl.row_offsets[b])
    J = np.asarray(J, dtype=np.int64) + off
    if wl.spec.kv_format == "bf16":
        return wl.rows_bf16[torch.from_numpy(J)].to(torch.float64).numpy()
    t = torch.from_numpy(J)
    return ofp8.dequant_rows(wl.nope_codes[t].numpy(), wl.scale_codes[t].numpy(),
                             wl.rope_bf16[t].to(torch.float64).numpy())


def oracle_of(wl, requests: Optional[Sequence[int]] = None, abs_mass: bool = False):
    """Oracle O [b, Sq, H, 512] and LSE [b, H, Sq] for the listed requests (all by default);
    with abs_mass also the weighted magnitude sum_j P_j |V_j| [b, Sq, H, 512]."""
    s = wl.spec
    req = list(range(s.batch)) if requests is None else list(requests)
    q = wl.q[req].to(torch.float64).numpy()
    seq = wl.seqlens[req]
    idx = None if wl.indices is None else wl.indices[req].numpy()
    tl = None
    if wl.topk_lens is not None:
        tl = wl.topk_lens.numpy().reshape(s.batch, s.q_len)[req].reshape(-1)
    sink = None if wl.sink is None else wl.sink.to(torch.float64).numpy()
    if idx is None:
        return oatt.mla_decode(q, lambda i: dense_rows(wl, req[i]), seq, s.sm_scale, s.d_v,
                               s.causal, s.window, None, None, sink, abs_mass)
    # index lists: decode only the listed rows of each (request, token)
    B, Sq, H = len(req), s.q_len, s.num_heads
    O = np.zeros((B, Sq, H, s.d_v))
    LSE = np.zeros((B, H, Sq))
    A = np.zeros((B, Sq, H, s.d_v))
    for i, b in enumerate(req):
        L = int(seq[i])
        for t in range(Sq):
            n = None if tl is None else int(tl[i * Sq + t])
            J = oatt.visible_sparse(L, idx[i, t], n)
            K = dense_rows_at(wl, b, J)
            o, l, a = oatt.attend(q[i, t], K, s.sm_scale, s.d_v, sink, abs_mass=True)
            O[i, t] = o
            LSE[i, :, t] = l
            A[i, t] = a
    return (O, LSE, A) if abs_mass else (O, LSE)


def plan_words(wl, num_cus: int) -> np.ndarray:
    s = wl.spec
    tl = None if wl.topk_lens is None else wl.topk_lens.numpy()
    return oplan.build_plan(wl.seqlens, s.q_len, s.num_heads, num_cus, s.topk, s.window, tl)


def check_split_descriptors(plan: torch.Tensor, want_words: np.ndarray, wl) -> None:
    """The plan's per-split descriptors (after the padded words and 9472 bytes of zero rows: one
    32-byte record per split, (g, b, j0, n, L, q0, qend, nsplit)) against the oracle plan's words
    they restate: the split record, the group's rows and split count, the request's length."""
    s = wl.spec
    w = np.asarray(want_words, dtype=np.int64)
    G, U, S = int(w[1]), int(w[2]), int(w[3])
    grp_ptr = w[16:16 + G + 1]
    grp_rows = w[16 + G + 1 + U + 1:16 + G + 1 + U + 1 + 2 * G].reshape(G, 2)
    recs = w[16 + G + 1 + U + 1 + 2 * G:][:4 * S].reshape(S, 4)
    n_words = 16 + (G + 1) + (U + 1) + 2 * G + 4 * (G + U)
    off = (n_words * 4 + 255) // 256 * 256 + 9472
    got = plan.numpy()[off:off + 32 * S].view(np.int32).reshape(S, 8)
    for sp in range(S):
        g, kb, ke = int(recs[sp, 0]), int(recs[sp, 1]), int(recs[sp, 2])
        j0, n = int(grp_rows[g, 0]), int(grp_rows[g, 1])
        b = g // s.q_len if s.topk > 0 else g
        want = [g, b, j0, n, int(wl.seqlens[b]), 2 * kb, min(2 * ke, -(-n // 32)),
                int(grp_ptr[g + 1] - grp_ptr[g])]
        assert got[sp].tolist() == want, f"split {sp}: descriptor {got[sp].tolist()} != {want}"


def metrics(out: torch.Tensor, lse: torch.Tensor, O_ref: np.ndarray, L_ref: np.ndarray,
            A_ref: Optional[np.ndarray] = None) -> dict:
    """Error metrics of a GPU result against the oracle.

    max_abs_scaled divides each output's error by max(1, A) where A = sum_j P_j |V_j|: the bf16
    probabilities the PV product runs on carry a relative rounding of 2^-9, so the absolute error
    of an output scales with the magnitude of its terms, not with |O| (terms of size 30 that cancel
    to |O| = 1 keep an error of order 0.06). For values of order one (bf16 rows drawn N(0,1)) the
    bound is the plain absolute one.
    """
    o = out.to(torch.float64).numpy()
    l = lse.to(torch.float64).numpy()
    diff = o - O_ref
    nref = np.linalg.norm(O_ref)
    finite_ref = np.isfinite(L_ref)
    lse_match_inf = bool(np.all(np.isneginf(l[~finite_ref]))) if (~finite_ref).any() else True
    lse_err = float(np.max(np.abs(l[finite_ref] - L_ref[finite_ref]))) if finite_ref.any() else 0.0
    return dict(
        rel_l2=float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff)),
        max_abs=float(np.max(np.abs(diff))) if diff.size else 0.0,
        max_abs_scaled=float(np.max(np.abs(diff) / np.maximum(1.0, np.abs(O_ref) if A_ref is None
                                                              else A_ref))) if diff.size else 0.0,
        lse_max_abs=lse_err,
        lse_inf_ok=lse_match_inf,
        finite=bool(np.all(np.isfinite(o))),
    )


def scaled_bound(wl) -> bool:
    """Whether the max-abs bar of a workload is taken relative to the term magnitudes.

    Only fp8 rows whose ue8m0 scale exponents are not all zero: their terms reach 2^4 x 448 and the
    bf16 rounding of the probabilities then leaves an error proportional to those terms (terms of
    size 30 that cancel to |O| = 1 keep an error of order 0.06). Every other case, bf16 rows and
    fp8 rows at exponent 0, is held to the plain bound |O - O_ref| <= 2e-2."""
    s = wl.spec
    return s.kv_format == "fp8" and tuple(s.scale_exp_range) != (0, 0)


def assert_parity(m: dict, rel_l2=REL_L2, max_abs=MAX_ABS, lse_abs=LSE_ABS, ctx="",
                  scaled: bool = False):
    """The parity bar: rel-L2, LSE and, per element, the plain max-abs bound (or, with scaled, the
    bound relative to max(1, sum_j P_j |V_j|)); the message carries both max-abs figures."""
    nums = f"max_abs={m['max_abs']:.3e} max_abs_scaled={m['max_abs_scaled']:.3e}"
    assert m["finite"], f"{ctx} non-finite outputs {m}"
    assert m["lse_inf_ok"], f"{ctx} empty rows must give LSE -inf {m}"
    assert m["rel_l2"] <= rel_l2, f"{ctx} rel-L2 {m}"
    if scaled:
        assert m["max_abs_scaled"] <= max_abs, f"{ctx} scaled max-abs ({nums}) {m}"
    else:
        assert m["max_abs"] <= max_abs, f"{ctx} max-abs ({nums}) {m}"
    assert m["lse_max_abs"] <= lse_abs, f"{ctx} LSE {m}"
