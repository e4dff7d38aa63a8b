"""The C ABI library (no GPU needed): it loads, exports every function include/mla.h declares, and
rejects invalid arguments on the host before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

import mla_paged_latent_plan_amd as mla
from mla_paged_latent_plan_amd import _lib, build

HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB_PATH):
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {build.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def good(**kw):
    base = dict(batch=2, q_len=1, num_heads=16, d_qk=576, kv_format=0, page_size=16,
                page_stride_bytes=16 * 1152, num_pages=10, max_pages_per_seq=8)
    base.update(kw)
    return mla.make_problem(**base)


def ws(p, cus=256):
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    return _lib.load().mla_get_workspace_size(ctypes.byref(p), cus, ctypes.byref(a),
                                              ctypes.byref(b)), a.value, b.value


def test_workspace_sizes(lib):
    rc, plan_b, part_b = ws(good(), 256)
    assert rc == 0
    G, U = 2, 256
    words = 16 + (G + 1) + (U + 1) + 2 * G + 4 * (G + U)
    # words, padded to 256 bytes, 9472 bytes of zero rows, then a 32-byte descriptor per split slot
    assert plan_b == ((words * 4 + 255) // 256) * 256 + 9472 + 32 * (G + U)
    assert part_b == (G + U) * 16 * (512 * 2 + 4)
    # 128 heads: one 128-row tile per group, U = cus
    rc, _, part_b = ws(good(num_heads=128), 256)
    assert rc == 0 and part_b == (2 + 256) * 128 * (512 * 2 + 4)
    # 4 tokens x 64 heads = 256 rows -> 2 tiles of 128, U = 128
    rc, _, part_b = ws(good(num_heads=64, q_len=4, causal=1, window=128), 256)
    assert rc == 0 and part_b == (2 + 128) * 256 * (512 * 2 + 4)
    # index lists: groups are (request, token) pairs of H rows
    rc, _, part_b = ws(good(num_heads=128, q_len=2, topk=64), 256)
    assert rc == 0 and part_b == (4 + 256) * 128 * (512 * 2 + 4)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 2), (dict(q_len=0), 2), (dict(num_heads=0), 2), (dict(d_qk=320), 2),
    (dict(d_v=448), 2), (dict(d_rope=32), 2), (dict(kv_format=2), 3), (dict(page_size=24), 4),
    (dict(page_size=0), 4), (dict(page_size=8192), 4), (dict(page_stride_bytes=100), 4),
    (dict(page_stride_bytes=16 * 1152 - 16), 4), (dict(num_pages=0), 4),
    (dict(max_pages_per_seq=0), 4), (dict(topk=-1), 5), (dict(window=-3), 5),
    (dict(causal=2), 5), (dict(topk=8, causal=1), 5), (dict(topk=8, window=4), 5),
    (dict(batch=9000, topk=4), 2),
    (dict(kv_format=1, page_stride_bytes=16 * 640), 4),
])
def test_invalid_problems_rejected(lib, kw, status):
    rc, _, _ = ws(good(**kw))
    assert rc == status, (kw, rc)


def test_fp8_layout_accepted(lib):
    rc, _, _ = ws(good(kv_format=1, page_stride_bytes=16 * 648))
    assert rc == 0
    rc, _, _ = ws(good(kv_format=1, d_qk=512, page_size=64, page_stride_bytes=37440))
    assert rc == 0


def test_host_checks_before_launch(lib):
    p = good()
    vp = ctypes.c_void_p
    # null seqlens / plan
    assert lib.mla_decode_plan(ctypes.byref(p), 256, None, None, vp(4096), 1 << 20, None) == 1
    assert lib.mla_decode_plan(ctypes.byref(p), 256, vp(4096), None, None, 1 << 20, None) == 1
    # misaligned plan, plan too small
    assert lib.mla_decode_plan(ctypes.byref(p), 256, vp(4096), None, vp(4100), 1 << 20, None) == 7
    assert lib.mla_decode_plan(ctypes.byref(p), 256, vp(4096), None, vp(4096), 64, None) == 6
    # decode: null q, bad scale, small partials
    args = [ctypes.byref(p), 256, None, vp(4096), vp(4096), vp(4096), ctypes.c_float(0.1), None,
            None, vp(4096), vp(4096), 1 << 30, vp(4096), vp(4096), None]
    assert lib.mla_decode(*args) == 1
    args[2] = vp(4096)
    args[6] = ctypes.c_float(-1.0)
    assert lib.mla_decode(*args) == 2
    args[6] = ctypes.c_float(0.1)
    args[11] = 16
    assert lib.mla_decode(*args) == 6
    # index lists without indices
    ps = good(topk=8)
    args[0] = ctypes.byref(ps)
    args[11] = 1 << 30
    assert lib.mla_decode(*args) == 1
    # combine: null out
    assert lib.mla_combine(ctypes.byref(p), 256, vp(4096), vp(4096), 1 << 30, None, None, vp(4096),
                           None) == 1
    assert lib.mla_strerror(6) == b"workspace buffer too small"


def test_kv_write_host_checks(lib):
    p = good()
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    # no tokens: nothing to check or enqueue
    assert lib.mla_kv_write(ctypes.byref(p), i64(0), None, None, None, None, None) == 0
    assert lib.mla_kv_write(ctypes.byref(p), i64(-1), vp(4096), vp(4096), vp(4096), vp(4096),
                            None) == 2
    assert lib.mla_kv_write(ctypes.byref(p), i64(4), None, vp(4096), vp(4096), vp(4096), None) == 1
    assert lib.mla_kv_write(ctypes.byref(p), i64(4), vp(4096), vp(4096), None, vp(4096), None) == 1
    # misaligned rows, misaligned slot mapping
    assert lib.mla_kv_write(ctypes.byref(p), i64(4), vp(4100), vp(4096), vp(4096), vp(4096),
                            None) == 7
    assert lib.mla_kv_write(ctypes.byref(p), i64(4), vp(4096), vp(4096), vp(4100), vp(4096),
                            None) == 7
    # an invalid problem is rejected first
    bad = good(page_size=24)
    assert lib.mla_kv_write(ctypes.byref(bad), i64(4), vp(4096), vp(4096), vp(4096), vp(4096),
                            None) == 4


def test_absorb_host_checks(lib):
    vp = ctypes.c_void_p
    # no tokens: nothing to check or enqueue
    assert lib.mla_q_absorb(0, 128, 128, 512, 64, None, None, None, None, None) == 0
    assert lib.mla_v_up(0, 128, 512, 128, None, None, None, None) == 0
    # shapes: negative tokens, k not a multiple of 32, columns not a multiple of 64, odd RoPE width
    assert lib.mla_q_absorb(-1, 128, 128, 512, 64, vp(4096), vp(4096), vp(4096), vp(4096), None) == 2
    assert lib.mla_q_absorb(4, 128, 100, 512, 64, vp(4096), vp(4096), vp(4096), vp(4096), None) == 2
    assert lib.mla_q_absorb(4, 128, 128, 500, 64, vp(4096), vp(4096), vp(4096), vp(4096), None) == 2
    assert lib.mla_q_absorb(4, 128, 128, 512, 60, vp(4096), vp(4096), vp(4096), vp(4096), None) == 2
    assert lib.mla_v_up(4, 128, 500, 128, vp(4096), vp(4096), vp(4096), None) == 2
    assert lib.mla_v_up(4, 128, 512, 100, vp(4096), vp(4096), vp(4096), None) == 2
    # null operands; q_pe may be NULL only without a RoPE part
    assert lib.mla_q_absorb(4, 128, 128, 512, 64, vp(4096), None, vp(4096), vp(4096), None) == 1
    assert lib.mla_q_absorb(4, 128, 128, 512, 64, vp(4096), vp(4096), None, vp(4096), None) == 1
    assert lib.mla_v_up(4, 128, 512, 128, None, vp(4096), vp(4096), None) == 1
    # alignment
    assert lib.mla_q_absorb(4, 128, 128, 512, 64, vp(4104), vp(4096), vp(4096), vp(4096), None) == 7
    assert lib.mla_v_up(4, 128, 512, 128, vp(4096), vp(4096), vp(4100), None) == 7


def test_swa_runs_host_checks(lib):
    vp = ctypes.c_void_p
    assert lib.mla_swa_runs(0, 128, None, None, 64, 1, None, None) == 0
    assert lib.mla_swa_runs(-1, 128, vp(4096), None, 64, 1, vp(4096), None) == 2
    assert lib.mla_swa_runs(4, 0, vp(4096), None, 64, 1, vp(4096), None) == 2
    assert lib.mla_swa_runs(4, 128, vp(4096), None, 48, 1, vp(4096), None) == 4
    assert lib.mla_swa_runs(4, 128, vp(4096), None, 64, 2, vp(4096), None) == 5
    assert lib.mla_swa_runs(4, 128, None, None, 64, 1, vp(4096), None) == 1
    assert lib.mla_swa_runs(4, 128, vp(4096), None, 64, 1, vp(4104), None) == 7
    assert lib.mla_swa_runs(4, 128, vp(4098), None, 64, 1, vp(4096), None) == 7


def test_gather_host_checks(lib):
    p = good()
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    assert lib.mla_gather_context(ctypes.byref(p), 1, i64(0), None, None, None, None, None, None,
                                  None) == 0
    assert lib.mla_gather_context(ctypes.byref(p), 0, i64(4), vp(4096), vp(4096), None, vp(4096),
                                  vp(4096), vp(4096), None) == 2
    assert lib.mla_gather_context(ctypes.byref(p), 1, i64(4), None, vp(4096), None, vp(4096),
                                  vp(4096), vp(4096), None) == 1
    assert lib.mla_gather_context(ctypes.byref(p), 1, i64(4), vp(4096), vp(4096), None, vp(4096),
                                  vp(4096), vp(4100), None) == 7


def test_planner_null_and_empty(lib):
    nc = np.zeros(1, dtype=np.int32)
    ptr = np.zeros(4, dtype=np.int32)
    assert lib.mla_plan_context_chunks(0, None, 64, 16, 4, 4, nc.ctypes.data, ptr.ctypes.data,
                                       None, None, None) == 0 and nc[0] == 0
    assert lib.mla_plan_context_chunks(2, None, 64, 16, 4, 4, nc.ctypes.data, ptr.ctypes.data,
                                       None, None, None) == 1


def test_sparse_prefill_host_checks(lib):
    """Workspace layout of the sparse prefill (metadata | plan | partials | split maxima, 256-byte
    aligned parts) and its argument checks; no launch happens on any failing call."""
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    n = ctypes.c_size_t(0)
    s_q, H, d_qk, topk, s_kv, cus = 300, 128, 576, 2048, 70000, 256
    assert lib.mla_sparse_prefill_workspace_size(s_q, H, d_qk, topk, i64(s_kv), cus, ctypes.byref(n)) == 0
    pages = (s_kv + 4095) // 4096
    p = mla.make_problem(1, s_q, H, d_qk, 0, 4096, 4096 * 2 * d_qk, pages, pages, topk=topk)
    rc, plan_b, part_b = ws(p, cus)
    assert rc == 0
    r256 = lambda x: (x + 255) // 256 * 256
    U = cus // ((H + 127) // 128)  # 128-row tiles above 64 heads
    expect = r256(r256(r256(4 * (1 + pages)) + plan_b) + part_b) + (s_q + U) * H * 4
    assert n.value == expect
    # sizes out of range
    for args in ((0, H, d_qk, topk, 5), (8193, H, d_qk, topk, 5), (4, H, d_qk, 0, 5),
                 (4, H, d_qk, topk, 0), (4, H, d_qk, topk, 2 ** 31), (4, H, 600, topk, 5),
                 (4, 0, d_qk, topk, 5)):
        assert lib.mla_sparse_prefill_workspace_size(*args[:4], i64(args[4]), cus, ctypes.byref(n)) == 2, args
    # nulls, alignment, scale, workspace size
    good_args = [4, 64, 512, 128, i64(1000), cus, vp(4096), vp(4096), vp(4096), 0.1, vp(4096),
                 1 << 30, vp(4096), vp(4096), vp(4096), None]
    def call(**change):
        a = list(good_args)
        for k, v in change.items():
            a[int(k[1:])] = v
        return lib.mla_sparse_prefill(*a)
    assert call(a6=None) == 1 and call(a8=None) == 1 and call(a13=None) == 1
    assert call(a10=None) == 1
    assert call(a7=vp(4100)) == 7 and call(a12=vp(4104)) == 7
    assert call(a9=0.0) == 2 and call(a9=float("nan")) == 2
    assert call(a11=16) == 6


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """mla_decode_noalloc: a problem whose plan and partials exceed the static scratch (512
    requests of 4 tokens x 64 heads on 256 CUs: about 151 MB of partials) is refused before
    anything is enqueued; NULL inputs are refused too."""
    p = good(batch=512, q_len=4, num_heads=64, d_qk=512, page_size=64, page_stride_bytes=64 * 1024,
             num_pages=10, max_pages_per_seq=8, causal=1, window=128)
    nz = ctypes.c_void_p(16)
    rc = lib.mla_decode_noalloc(ctypes.byref(p), 256, nz, nz, nz, nz, None, 0.1, None, None, nz,
                                nz, None)
    assert rc == 10 and lib.mla_strerror(rc).decode().startswith("plan and partials exceed")
    small = good()
    rc = lib.mla_decode_noalloc(ctypes.byref(small), 256, None, nz, nz, nz, None, 0.1, None, None,
                                nz, nz, None)
    assert rc == 1
