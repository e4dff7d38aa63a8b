"""ctypes binding of libmla.so — argument marshalling only; every step runs in the HIP kernels.

Function names mirror the C ABI of include/mla.h. Torch supplies device memory and the current
stream; tensors are passed by data pointer after host-side dtype/shape/device checks.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

from .build import LIB_PATH

MLA_KV_BF16 = 0
MLA_KV_FP8 = 1

STATUS = {
    0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_FORMAT", 4: "MLA_ERR_PAGE",
    5: "MLA_ERR_MODE", 6: "MLA_ERR_WORKSPACE", 7: "MLA_ERR_ALIGN", 8: "MLA_ERR_DEVICE",
    9: "MLA_ERR_LAUNCH", 10: "MLA_ERR_SCRATCH",
}

EXPORTS = ("mla_get_workspace_size", "mla_device_num_cus", "mla_decode_plan", "mla_decode",
           "mla_combine", "mla_decode_noalloc", "mla_kv_write", "mla_q_absorb", "mla_v_up", "mla_swa_runs", "mla_gather_context", "mla_plan_context_chunks",
           "mla_sparse_prefill_workspace_size", "mla_sparse_prefill", "mla_build_id",
           "mla_check_enable", "mla_check_status", "mla_strerror")


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Problem(ctypes.Structure):
    """struct mla_problem."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("page_stride_bytes", ctypes.c_int64),
        ("num_pages", ctypes.c_int64),
        ("max_pages_per_seq", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (built in-tree). Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(or python -m mla_paged_latent_plan_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.mla_get_workspace_size.argtypes = [P, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_device_num_cus.argtypes = [ctypes.POINTER(i32)]
    lib.mla_decode_plan.argtypes = [P, i32, vp, vp, vp, sz, vp]
    lib.mla_decode.argtypes = [P, i32, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp, vp,
                               vp]
    lib.mla_combine.argtypes = [P, i32, vp, vp, sz, vp, vp, vp, vp]
    lib.mla_decode_noalloc.argtypes = [P, i32, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                       vp]
    lib.mla_kv_write.argtypes = [P, ctypes.c_int64, vp, vp, vp, vp, vp]
    lib.mla_q_absorb.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.mla_v_up.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
    lib.mla_swa_runs.argtypes = [i32, i32, vp, vp, i32, i32, vp, vp]
    lib.mla_gather_context.argtypes = [P, i32, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp]
    lib.mla_plan_context_chunks.argtypes = [i32, vp, ctypes.c_int64, i32, i32, i32, vp, vp, vp, vp,
                                            vp]
    i64 = ctypes.c_int64
    lib.mla_sparse_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i64, i32,
                                                      ctypes.POINTER(sz)]
    lib.mla_sparse_prefill.argtypes = [i32, i32, i32, i32, i64, i32, vp, vp, vp, ctypes.c_float,
                                       vp, sz, vp, vp, vp, vp]
    lib.mla_strerror.argtypes = [ctypes.c_int]
    lib.mla_strerror.restype = ctypes.c_char_p
    lib.mla_check_enable.argtypes = [i32]
    lib.mla_check_status.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32, vp]
    lib.mla_build_id.argtypes = []
    lib.mla_build_id.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("mla_strerror", "mla_build_id"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        msg = load().mla_strerror(status).decode()
        raise MLAError(fn, status, msg)


def workspace_size(p: Problem, num_cus: int):
    lib = load()
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    check("mla_get_workspace_size", lib.mla_get_workspace_size(ctypes.byref(p), num_cus,
                                                              ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def check_enable(on: bool) -> None:
    """Checked mode on or off for every later decode call (mla_check_enable)."""
    check("mla_check_enable", load().mla_check_enable(1 if on else 0))


def check_status(clear: bool, stream: int) -> int:
    """The current device's checked-mode bits after the stream's work (mla_check_status)."""
    bits = ctypes.c_uint32(0)
    check("mla_check_status", load().mla_check_status(ctypes.byref(bits), 1 if clear else 0,
                                                      ctypes.c_void_p(stream)))
    return int(bits.value)


def device_num_cus() -> int:
    n = ctypes.c_int32(0)
    check("mla_device_num_cus", load().mla_device_num_cus(ctypes.byref(n)))
    return n.value


def build_id() -> str:
    """The source hash the loaded libmla.so was built from (mla_build_id)."""
    return load().mla_build_id().decode()


def check_build_id() -> str:
    """Raise unless the loaded library was built from the sources in this tree; returns the id."""
    from .build import source_id
    got, want = build_id(), source_id()
    if got != want:
        raise ImportError(f"libmla.so was built from other sources (build id {got}, sources {want}): "
                          "rebuild it with __graft_entry__.build()")
    return got
