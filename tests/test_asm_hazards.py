"""MFMA result hazards in the generated gfx950 code.

The decode and absorb kernels issue their MFMAs as inline assembly (to pin accumulators to VGPRs or
AGPRs), so the compiler's hazard recogniser does not know that those instructions write their
destination registers several cycles after they issue. Every read of an MFMA result is therefore
preceded by explicit wait states in the source. The compiler can still place an instruction of its
own (a register copy for a tied asm operand, say) between an MFMA and that wait; such an instruction
reads a stale value. This test compiles the kernels to assembly and checks that no instruction other
than an MFMA touches an MFMA destination register within 18 wait states of the MFMA (an XDL
16x16x32 result needs fewer than that before a VALU may read or overwrite it).
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from mla_paged_latent_plan_amd import build as B

WINDOW = 18


def _regs(tok):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", tok):
        if m.group(5):
            out.add((m.group(4), int(m.group(5))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def scan(asm: str):
    """(kernel, line, mfma, offending instruction) for every instruction that reads or writes an
    MFMA destination register fewer than WINDOW wait states after the MFMA, within a basic block."""
    hits = []
    for km in re.finditer(r"^(_Z\w+):", asm, re.M):
        name = km.group(1)
        end = asm.find(".Lfunc_end", km.end())
        lines = [l.strip() for l in asm[km.end():end].split("\n")]
        for n, l in enumerate(lines):
            if not l.startswith("v_mfma"):
                continue
            dst = _regs(l.split(None, 1)[1].split(",")[0])
            ws = 0
            for t in lines[n + 1:n + 200]:
                if not t or t.startswith((";", ".")):
                    if t.startswith(".LBB"):
                        break  # a block boundary: the checks stop here (waits sit before branches)
                    continue
                op = t.split()[0]
                if op == "s_nop":
                    ws += int(t.split()[1], 0) + 1
                elif op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                    break
                else:
                    args = t.split(None, 1)[1] if len(t.split(None, 1)) > 1 else ""
                    if op.startswith("v_mfma"):
                        # a following MFMA may accumulate onto the same registers (srcC = vdst)
                        parts = args.split(",")
                        rd = set()
                        for p in parts[1:3]:
                            rd |= _regs(p)
                        if rd & dst:
                            hits.append((name, n, l, t))
                    elif _regs(args) & dst:
                        hits.append((name, n, l, t))
                    ws += 1
                if ws >= WINDOW:
                    break
    return hits


def _compile(src: str, out: str, inc: str):
    cmd = [B.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, src, "-o", out]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


needs_hipcc = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                 reason="hipcc not available")


@needs_hipcc
def test_scanner_flags_an_early_read():
    """The scanner itself: an MFMA result read at once is flagged, the same read after the wait
    states is not."""
    src = r"""
#include <hip/hip_runtime.h>
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
template <int NOP>
__global__ void k(float* p, bf16x8 a, bf16x8 b) {
  f32x4 c;
  float r;
  if constexpr (NOP)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3\n\tv_mov_b32 %1, %0"
                 : "=&v"(c), "=v"(r) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\tv_mov_b32 %1, %0" : "=&v"(c), "=v"(r) : "v"(a), "v"(b));
  p[threadIdx.x] = r;
}
template __global__ void k<0>(float*, bf16x8, bf16x8);
template __global__ void k<1>(float*, bf16x8, bf16x8);
"""
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "probe.hip")
        with open(path, "w") as f:
            f.write(src)
        p = _compile(path, os.path.join(d, "probe.s"), B.CSRC)
        _, err = p.communicate()
        assert p.returncode == 0, err
        with open(os.path.join(d, "probe.s")) as f:
            hits = scan(f.read())
    names = {h[0] for h in hits}
    assert any("ILi0E" in n for n in names), hits
    assert not any("ILi1E" in n for n in names), hits


@needs_hipcc
def test_no_early_mfma_result_access():
    with tempfile.TemporaryDirectory() as d:
        procs = {}
        for f in ("decode.hip", "absorb.hip"):
            procs[f] = _compile(os.path.join(B.CSRC, f), os.path.join(d, f + ".s"), B.CSRC)
        problems = []
        for f, p in procs.items():
            _, err = p.communicate()
            assert p.returncode == 0, err[-2000:]
            with open(os.path.join(d, f + ".s")) as fh:
                hits = scan(fh.read())
            problems += [f"{f}: {k}: {m} -> {t}" for (k, _, m, t) in hits]
    assert not problems, "\n".join(problems[:20])
