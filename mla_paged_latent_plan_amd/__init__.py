"""MI355X (gfx950) MLA decode over a paged latent KV cache.

Thin Python layer over libmla.so (include/mla.h): plan, decode and combine with the same names as
the C ABI. Torch provides device memory and the current HIP stream; the computation is entirely in
the HIP kernels, and the functions fail loudly when the library is missing or a tensor does not
match the problem.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import MLA_KV_BF16, MLA_KV_FP8, MLAError, Problem  # noqa: F401

__all__ = ["Problem", "make_problem", "workspace_size", "mla_decode_plan", "mla_decode",
           "mla_combine", "mla_decode_noalloc", "mla_kv_write", "mla_q_absorb", "mla_v_up", "mla_swa_runs", "mla_gather_context", "plan_context_chunks",
           "sparse_prefill_workspace_size", "mla_sparse_prefill", "MLADecode", "device_num_cus",
           "MLAError"]


def device_num_cus() -> int:
    return _lib.device_num_cus()


def make_problem(batch: int, q_len: int, num_heads: int, d_qk: int, kv_format: int,
                 page_size: int, page_stride_bytes: int, num_pages: int, max_pages_per_seq: int,
                 topk: int = 0, causal: bool = False, window: int = 0, d_v: int = 512,
                 d_rope: int = 64) -> Problem:
    return Problem(batch, q_len, num_heads, d_qk, d_v, d_rope, kv_format, page_size,
                   page_stride_bytes, num_pages, max_pages_per_seq, topk, int(causal), window)


def workspace_size(p: Problem, num_cus: int):
    """(plan_bytes, partial_bytes) for a problem planned over num_cus compute units."""
    return _lib.workspace_size(p, num_cus)


def _ptr(t: Optional[torch.Tensor], dtype, name: str, numel: Optional[int] = None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


MLA_CHECK_PAGE, MLA_CHECK_LENGTH, MLA_CHECK_PLAN = 1, 2, 4


def mla_check_enable(on: bool) -> None:
    """Checked mode for every later decode call: a validation kernel records contract violations
    (MLA_CHECK_* bits) in a per-device word (include/mla.h, mla_check_enable)."""
    _lib.check_enable(on)


def mla_check_status(clear: bool = True, stream=None) -> int:
    """The current device's MLA_CHECK_* bits once the stream's work is done (mla_check_status)."""
    return _lib.check_status(clear, _stream(stream))


def mla_decode_plan(p: Problem, num_cus: int, seqlens: torch.Tensor,
                    topk_lens: Optional[torch.Tensor], plan: torch.Tensor, stream=None) -> None:
    lib = _lib.load()
    _lib.check("mla_decode_plan", lib.mla_decode_plan(
        p, num_cus, _ptr(seqlens, torch.int32, "seqlens", p.batch),
        _ptr(topk_lens, torch.int32, "topk_lens", p.batch * p.q_len), _ptr(plan, torch.uint8, "plan"),
        plan.numel(), _stream(stream)))


def mla_decode(p: Problem, num_cus: int, q: torch.Tensor, kv_cache: torch.Tensor,
               block_table: torch.Tensor, seqlens: torch.Tensor, sm_scale: float,
               indices: Optional[torch.Tensor], sink: Optional[torch.Tensor], plan: torch.Tensor,
               partials: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, stream=None) -> None:
    lib = _lib.load()
    B, Sq, H = p.batch, p.q_len, p.num_heads
    if tuple(q.shape) != (B, Sq, H, p.d_qk):
        raise ValueError(f"q must be [{B}, {Sq}, {H}, {p.d_qk}], got {tuple(q.shape)}")
    if tuple(out.shape) != (B, Sq, H, p.d_v):
        raise ValueError(f"out must be [{B}, {Sq}, {H}, {p.d_v}], got {tuple(out.shape)}")
    if kv_cache.numel() < p.num_pages * p.page_stride_bytes // kv_cache.element_size():
        raise ValueError("kv_cache is smaller than num_pages * page_stride_bytes")
    if tuple(block_table.shape) != (B, p.max_pages_per_seq):
        raise ValueError("block_table must be [batch, max_pages_per_seq]")
    if p.topk > 0 and (indices is None or tuple(indices.shape) != (B, Sq, p.topk)):
        raise ValueError("indices must be [batch, q_len, topk] when topk > 0")
    _lib.check("mla_decode", lib.mla_decode(
        p, num_cus, _ptr(q, torch.bfloat16, "q"), kv_cache.data_ptr(),
        _ptr(block_table, torch.int32, "block_table"), _ptr(seqlens, torch.int32, "seqlens", B),
        float(sm_scale), _ptr(indices, torch.int32, "indices"), _ptr(sink, torch.float32, "sink", H),
        _ptr(plan, torch.uint8, "plan"), _ptr(partials, torch.uint8, "partials"), partials.numel(),
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse", B * H * Sq),
        _stream(stream)))


def mla_combine(p: Problem, num_cus: int, plan: torch.Tensor, partials: torch.Tensor,
                sink: Optional[torch.Tensor], out: torch.Tensor, lse: torch.Tensor,
                stream=None) -> None:
    lib = _lib.load()
    B, Sq, H = p.batch, p.q_len, p.num_heads
    if tuple(out.shape) != (B, Sq, H, p.d_v):
        raise ValueError(f"out must be [{B}, {Sq}, {H}, {p.d_v}], got {tuple(out.shape)}")
    if lse.numel() != B * H * Sq:
        raise ValueError(f"lse must hold [{B}, {H}, {Sq}], got {tuple(lse.shape)}")
    _lib.check("mla_combine", lib.mla_combine(
        p, num_cus, _ptr(plan, torch.uint8, "plan"), _ptr(partials, torch.uint8, "partials"),
        partials.numel(), _ptr(sink, torch.float32, "sink", p.num_heads),
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse", B * H * Sq),
        _stream(stream)))


def mla_decode_noalloc(p: Problem, num_cus: int, q: torch.Tensor, kv_cache: torch.Tensor,
                       block_table: torch.Tensor, seqlens: torch.Tensor,
                       topk_lens: Optional[torch.Tensor], sm_scale: float,
                       indices: Optional[torch.Tensor], sink: Optional[torch.Tensor],
                       out: torch.Tensor, lse: torch.Tensor, stream=None) -> None:
    """plan + decode + combine with the plan and partials in the library's static device scratch
    (no buffer of the caller's beyond inputs and outputs)."""
    lib = _lib.load()
    B, Sq, H = p.batch, p.q_len, p.num_heads
    if tuple(q.shape) != (B, Sq, H, p.d_qk):
        raise ValueError(f"q must be [{B}, {Sq}, {H}, {p.d_qk}], got {tuple(q.shape)}")
    if tuple(out.shape) != (B, Sq, H, p.d_v):
        raise ValueError(f"out must be [{B}, {Sq}, {H}, {p.d_v}], got {tuple(out.shape)}")
    if kv_cache.numel() < p.num_pages * p.page_stride_bytes // kv_cache.element_size():
        raise ValueError("kv_cache is smaller than num_pages * page_stride_bytes")
    if tuple(block_table.shape) != (B, p.max_pages_per_seq):
        raise ValueError("block_table must be [batch, max_pages_per_seq]")
    if p.topk > 0 and (indices is None or tuple(indices.shape) != (B, Sq, p.topk)):
        raise ValueError("indices must be [batch, q_len, topk] when topk > 0")
    _lib.check("mla_decode_noalloc", lib.mla_decode_noalloc(
        p, num_cus, _ptr(q, torch.bfloat16, "q"), kv_cache.data_ptr(),
        _ptr(block_table, torch.int32, "block_table"), _ptr(seqlens, torch.int32, "seqlens", B),
        _ptr(topk_lens, torch.int32, "topk_lens", B * Sq), float(sm_scale),
        _ptr(indices, torch.int32, "indices"), _ptr(sink, torch.float32, "sink", H),
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse", B * H * Sq),
        _stream(stream)))


def mla_kv_write(p: Problem, kv_c: torch.Tensor, k_pe: torch.Tensor, slot_mapping: torch.Tensor,
                 kv_cache: torch.Tensor, stream=None) -> None:
    """Write each token's [kv_c, k_pe] row into its cache slot (fp8 caches: quantised)."""
    lib = _lib.load()
    n = int(kv_c.shape[0]) if kv_c.dim() == 2 else -1
    if tuple(kv_c.shape) != (n, p.d_qk - p.d_rope):
        raise ValueError(f"kv_c must be [n, {p.d_qk - p.d_rope}], got {tuple(kv_c.shape)}")
    if tuple(k_pe.shape) != (n, p.d_rope):
        raise ValueError(f"k_pe must be [{n}, {p.d_rope}], got {tuple(k_pe.shape)}")
    if tuple(slot_mapping.shape) != (n,):
        raise ValueError(f"slot_mapping must be [{n}], got {tuple(slot_mapping.shape)}")
    if kv_cache.numel() * kv_cache.element_size() < p.num_pages * p.page_stride_bytes:
        raise ValueError("kv_cache is smaller than num_pages * page_stride_bytes")
    if not kv_cache.is_contiguous() or not kv_cache.is_cuda:
        raise ValueError("kv_cache must be a contiguous device tensor")
    _lib.check("mla_kv_write", lib.mla_kv_write(
        p, n, _ptr(kv_c, torch.bfloat16, "kv_c"), _ptr(k_pe, torch.bfloat16, "k_pe"),
        _ptr(slot_mapping, torch.int64, "slot_mapping"), kv_cache.data_ptr(), _stream(stream)))


def mla_q_absorb(q_nope: torch.Tensor, q_pe: Optional[torch.Tensor], w_uk: torch.Tensor,
                 q_out: torch.Tensor, stream=None) -> None:
    """q_out[t, h] = [q_nope[t, h] @ w_uk[h].T, q_pe[t, h]] (q_nope [T, H, P], w_uk [H, L, P])."""
    lib = _lib.load()
    T, H, P = q_nope.shape
    L = int(w_uk.shape[1])
    R = 0 if q_pe is None else int(q_pe.shape[2])
    if tuple(w_uk.shape) != (H, L, P):
        raise ValueError(f"w_uk must be [{H}, L, {P}], got {tuple(w_uk.shape)}")
    if q_pe is not None and tuple(q_pe.shape) != (T, H, R):
        raise ValueError(f"q_pe must be [{T}, {H}, R], got {tuple(q_pe.shape)}")
    if q_out.numel() != T * H * (L + R) or q_out.shape[-1] != L + R:
        raise ValueError(f"q_out must hold [{T}, {H}, {L + R}], got {tuple(q_out.shape)}")
    _lib.check("mla_q_absorb", lib.mla_q_absorb(
        T, H, P, L, R, _ptr(q_nope, torch.bfloat16, "q_nope"), _ptr(q_pe, torch.bfloat16, "q_pe"),
        _ptr(w_uk, torch.bfloat16, "w_uk"), _ptr(q_out, torch.bfloat16, "q_out", T * H * (L + R)),
        _stream(stream)))


def mla_v_up(o: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out[t, h] = o[t, h] @ w_uv[h].T (o [T, H, L], w_uv [H, V, L], out [T, H, V])."""
    lib = _lib.load()
    o3 = o.reshape(-1, o.shape[-2], o.shape[-1])
    T, H, L = o3.shape
    V = int(w_uv.shape[1])
    if tuple(w_uv.shape) != (H, V, L):
        raise ValueError(f"w_uv must be [{H}, V, {L}], got {tuple(w_uv.shape)}")
    if out.numel() != T * H * V:
        raise ValueError(f"out must hold [{T}, {H}, {V}], got {tuple(out.shape)}")
    _lib.check("mla_v_up", lib.mla_v_up(
        T, H, L, V, _ptr(o3, torch.bfloat16, "o"), _ptr(w_uv, torch.bfloat16, "w_uv"),
        _ptr(out, torch.bfloat16, "out"), _stream(stream)))


def mla_swa_runs(kv_indices: torch.Tensor, topk_lengths: Optional[torch.Tensor], page_size: int,
                 kv_run_step: int, runs: torch.Tensor, stream=None) -> None:
    """runs[t] = (slot0, len0, slot1, rows): token t's window of slots as at most two runs."""
    lib = _lib.load()
    T, topk = kv_indices.shape
    if tuple(runs.shape) != (T, 4):
        raise ValueError(f"runs must be [{T}, 4], got {tuple(runs.shape)}")
    _lib.check("mla_swa_runs", lib.mla_swa_runs(
        T, topk, _ptr(kv_indices, torch.int32, "kv_indices"),
        _ptr(topk_lengths, torch.int32, "topk_lengths", T), int(page_size), int(kv_run_step),
        _ptr(runs, torch.int32, "runs"), _stream(stream)))


def mla_gather_context(p: Problem, block_table: torch.Tensor, cu_seq_lens: torch.Tensor,
                       seq_starts: Optional[torch.Tensor], token_to_seq: torch.Tensor,
                       kv_cache: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst[i] = row seq_starts[r] + i - cu_seq_lens[r] of request r = token_to_seq[i], as bf16."""
    lib = _lib.load()
    n = int(token_to_seq.numel())
    R = int(block_table.shape[0])
    if tuple(block_table.shape) != (R, p.max_pages_per_seq):
        raise ValueError("block_table must be [num_reqs, max_pages_per_seq]")
    if cu_seq_lens.numel() != R + 1 or (seq_starts is not None and seq_starts.numel() != R):
        raise ValueError("cu_seq_lens must hold num_reqs + 1 entries, seq_starts num_reqs")
    if dst.numel() < n * p.d_qk:
        raise ValueError(f"dst must hold [{n}, {p.d_qk}]")
    if kv_cache.numel() * kv_cache.element_size() < p.num_pages * p.page_stride_bytes:
        raise ValueError("kv_cache is smaller than num_pages * page_stride_bytes")
    _lib.check("mla_gather_context", lib.mla_gather_context(
        p, R, n, _ptr(block_table, torch.int32, "block_table"),
        _ptr(cu_seq_lens, torch.int32, "cu_seq_lens"), _ptr(seq_starts, torch.int32, "seq_starts"),
        _ptr(token_to_seq, torch.int32, "token_to_seq"), kv_cache.data_ptr(),
        _ptr(dst, torch.bfloat16, "dst"), _stream(stream)))


def sparse_prefill_workspace_size(s_q: int, num_heads: int, d_qk: int, topk: int, s_kv: int,
                                  num_cus: int) -> int:
    """Workspace bytes of mla_sparse_prefill for these sizes."""
    import ctypes
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    _lib.check("mla_sparse_prefill_workspace_size", lib.mla_sparse_prefill_workspace_size(
        int(s_q), int(num_heads), int(d_qk), int(topk), int(s_kv), int(num_cus), ctypes.byref(n)))
    return n.value


def mla_sparse_prefill(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                       workspace: torch.Tensor, out: torch.Tensor, max_logits: torch.Tensor,
                       lse: torch.Tensor, num_cus: int, stream=None) -> None:
    """q [s_q, H, d_qk], kv [s_kv, d_qk] bf16, indices int32 [s_q, topk] -> out bf16 [s_q, H, 512],
    max_logits and lse fp32 [H, s_q] (flash_mla_sparse_fwd's outputs)."""
    lib = _lib.load()
    s_q, H, d_qk = q.shape
    s_kv = int(kv.shape[0])
    if kv.dim() != 2 or int(kv.shape[1]) != d_qk:
        raise ValueError(f"kv must be [s_kv, {d_qk}]")
    if indices.dim() != 2 or int(indices.shape[0]) != s_q:
        raise ValueError(f"indices must be [{s_q}, topk]")
    topk = int(indices.shape[1])
    if tuple(out.shape) != (s_q, H, 512) or tuple(max_logits.shape) != (H, s_q) or \
            tuple(lse.shape) != (H, s_q):
        raise ValueError("out must be [s_q, H, 512], max_logits and lse [H, s_q]")
    ws_bytes = workspace.numel() * workspace.element_size()
    _lib.check("mla_sparse_prefill", lib.mla_sparse_prefill(
        s_q, H, d_qk, topk, s_kv, int(num_cus), _ptr(q, torch.bfloat16, "q"),
        _ptr(kv, torch.bfloat16, "kv"), _ptr(indices, torch.int32, "indices"), float(sm_scale),
        _ptr(workspace, workspace.dtype, "workspace"), ws_bytes, _ptr(out, torch.bfloat16, "out"),
        _ptr(max_logits, torch.float32, "max_logits"), _ptr(lse, torch.float32, "lse"),
        _stream(stream)))


def plan_context_chunks(context_lens, workspace_rows: int, alignment: int):
    """Host plan of the chunked-context gather: a list of chunks, each a list of
    (request, first row, rows) spans (mla_plan_context_chunks)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    R = int(lens.size)
    total = int(np.maximum(lens, 0).sum())
    max_chunks = total // max(1, workspace_rows // alignment * alignment) + R + 2
    max_spans = R + max_chunks
    chunk_ptr = np.zeros(max_chunks + 1, dtype=np.int32)
    req, start, ln = (np.zeros(max_spans, dtype=np.int32) for _ in range(3))
    nc = np.zeros(1, dtype=np.int32)
    lib = _lib.load()
    addr = lambda a: a.ctypes.data
    _lib.check("mla_plan_context_chunks", lib.mla_plan_context_chunks(
        R, addr(lens) if R else None, int(workspace_rows), int(alignment), max_chunks, max_spans,
        addr(nc), addr(chunk_ptr), addr(req), addr(start), addr(ln)))
    return [[(int(req[k]), int(start[k]), int(ln[k])) for k in range(chunk_ptr[c], chunk_ptr[c + 1])]
            for c in range(int(nc[0]))]


class MLADecode:
    """Holds the plan and partial buffers of one problem and runs plan -> decode -> combine."""

    def __init__(self, p: Problem, num_cus: Optional[int] = None, device="cuda"):
        self.p = p
        self.num_cus = device_num_cus() if num_cus is None else int(num_cus)
        plan_bytes, part_bytes = workspace_size(p, self.num_cus)
        self.plan = torch.empty(plan_bytes, dtype=torch.uint8, device=device)
        self.partials = torch.empty(part_bytes, dtype=torch.uint8, device=device)

    def plan_(self, seqlens: torch.Tensor, topk_lens: Optional[torch.Tensor] = None, stream=None):
        mla_decode_plan(self.p, self.num_cus, seqlens, topk_lens, self.plan, stream)

    def decode_(self, q, kv_cache, block_table, seqlens, sm_scale, out, lse, indices=None,
                sink=None, stream=None):
        mla_decode(self.p, self.num_cus, q, kv_cache, block_table, seqlens, sm_scale, indices, sink,
                   self.plan, self.partials, out, lse, stream)
        mla_combine(self.p, self.num_cus, self.plan, self.partials, sink, out, lse, stream)

    def __call__(self, q, kv_cache, block_table, seqlens, sm_scale, indices=None, sink=None,
                 topk_lens=None, stream=None):
        p = self.p
        out = torch.empty(p.batch, p.q_len, p.num_heads, p.d_v, dtype=torch.bfloat16,
                          device=q.device)
        lse = torch.empty(p.batch, p.num_heads, p.q_len, dtype=torch.float32, device=q.device)
        self.plan_(seqlens, topk_lens, stream)
        self.decode_(q, kv_cache, block_table, seqlens, sm_scale, out, lse, indices, sink, stream)
        return out, lse
