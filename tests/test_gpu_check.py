"""Checked mode (include/mla.h, mla_check_enable / mla_check_status): with checks on, a
validation kernel runs before each decode and records violations of the data contract as bits of
a per-device word; the decode itself runs as before (out-of-range pages are read as zero rows)."""

import math

import pytest
import torch

from workloads import Spec, make

import mla_harness as H

pytestmark = pytest.mark.gpu

S = 1.0 / math.sqrt(192.0)
DENSE = Spec("check_dense", batch=3, q_len=1, num_heads=16, page_size=16, seqlens=(40, 1, 300),
             sm_scale=S, seed=50)
SPARSE = Spec("check_sparse", batch=2, q_len=2, num_heads=16, page_size=16, seqlens=(400, 90),
              topk=64, sm_scale=S, seed=51)
TILE128 = Spec("check_h128", batch=2, q_len=1, num_heads=128, page_size=64, seqlens=(700, 65),
               sm_scale=S, seed=52)


@pytest.fixture
def mla_checked():
    import mla_paged_latent_plan_amd as mla
    mla.mla_check_enable(True)
    mla.mla_check_status(clear=True)
    try:
        yield mla
    finally:
        mla.mla_check_enable(False)
        mla.mla_check_status(clear=True)


@pytest.mark.parametrize("spec", [DENSE, SPARSE, TILE128], ids=lambda s: s.name)
def test_valid_inputs_set_no_bits(mla_checked, spec):
    wl = make(spec)
    print(f"[gpu] checked mode, valid inputs: {spec.name}", flush=True)
    out, lse, _, _ = H.run_gpu(wl)
    assert mla_checked.mla_check_status() == 0
    O, L, A = H.oracle_of(wl, abs_mass=True)
    H.assert_parity(H.metrics(out, lse, O, L, A), ctx=f"checked {spec.name}")


@pytest.mark.parametrize("spec", [DENSE, TILE128], ids=lambda s: s.name)
def test_page_out_of_range_dense(mla_checked, spec):
    wl = make(spec)
    wl.block_table[0, 0] = wl.num_pages + 7  # page 0 of request 0 holds its first rows
    print(f"[gpu] checked mode, block-table entry past num_pages: {spec.name}", flush=True)
    H.run_gpu(wl)
    assert mla_checked.mla_check_status() == mla_checked.MLA_CHECK_PAGE


def test_page_out_of_range_index_list(mla_checked):
    wl = make(SPARSE)
    j = int(wl.indices[0, 0, 0])  # a listed row of request 0, token 0
    assert 0 <= j < int(wl.seqlens[0])
    wl.block_table[0, j // SPARSE.page_size] = -3
    print("[gpu] checked mode, negative block-table entry under an index list", flush=True)
    H.run_gpu(wl)
    assert mla_checked.mla_check_status() == mla_checked.MLA_CHECK_PAGE


def test_unused_bad_entry_and_checks_off(mla_checked):
    mla = mla_checked
    wl = make(DENSE)
    # request 1 has one row: its second page holds none, so a bad entry there is outside the contract
    wl.block_table[1, 1] = -1
    print("[gpu] checked mode, bad entry on an unused page", flush=True)
    H.run_gpu(wl)
    assert mla.mla_check_status() == 0
    wl.block_table[0, 0] = -1
    mla.mla_check_enable(False)
    print("[gpu] checks off, bad entry on a used page", flush=True)
    H.run_gpu(wl)
    assert mla.mla_check_status() == 0


def test_plan_of_another_problem(mla_checked):
    mla = mla_checked
    wl = make(DENSE)
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
    print("[gpu] checked mode, plan of another CU count", flush=True)
    mla.mla_decode_plan(p, 1, dev.seqlens, None, plan)
    mla.mla_decode(p, cus, dev.q, dev.cache, dev.block_table, dev.seqlens, s.sm_scale, None, None,
                   plan, partials, out, lse)
    assert mla.mla_check_status() == mla.MLA_CHECK_PLAN
