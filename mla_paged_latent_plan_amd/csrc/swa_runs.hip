// mla_swa_runs kernel: each token's sliding window of cache slots compressed into at most two runs
// (HALOps MLA API, mla_attention_plan). With s_g the slot of row g, rows g - 1 and g share a run iff
// s_g == s_{g-1} + kv_run_step and both lie on one page; a window with more than two runs (padding
// or not yet written) is described by its row 0 alone. Output per token: (slot0, len0, slot1,
// rows) — rows g < len0 at slot0 + step * g, the others at slot1 + step * (g - len0); slot1 = -1
// without a second run; an empty window is (-1, 0, -1, 0).
//
// One wave per token: lane l tests row g0 + l of each 64-row chunk for a run start (a slot that
// does not continue the previous one, or a page change, page = slot >> log2(page_size), i.e. floor
// division also for negative padding slots); a ballot gives the chunk's starts, the first start is
// the lowest set bit, and the wave stops once two starts are seen.
#include "layer_internal.h"

namespace mla {

namespace {

constexpr int kTokensPerBlock = 4;

__global__ __launch_bounds__(256) void swa_runs_kernel(SwaRunsArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
  if (t >= a.T) return;
  int n = a.topk;
  if (a.lengths != nullptr) n = min(max(a.lengths[t], 0), a.topk);
  const int32_t* kv = a.kv + t * a.topk;
  int out[4] = {-1, 0, -1, 0};
  if (n > 0) {
    int starts = 0, first = n;
    for (int g0 = 0; g0 < n && starts < 2; g0 += 64) {
      const int g = g0 + lane;
      bool brk = false;
      if (g >= 1 && g < n) {
        const int cur = kv[g], prev = kv[g - 1];
        brk = ((int64_t)cur != (int64_t)prev + a.step) || ((cur >> a.ps_log2) != (prev >> a.ps_log2));
      }
      const uint64_t m = __ballot(brk);
      if (m != 0 && starts == 0) first = g0 + __builtin_ctzll(m);
      starts += __popcll(m);
    }
    const int s0 = kv[0];
    if (starts == 0) {
      out[0] = s0; out[1] = n; out[2] = -1; out[3] = n;
    } else if (starts == 1) {
      out[0] = s0; out[1] = first; out[2] = kv[first]; out[3] = n;
    } else {
      out[0] = s0; out[1] = 1; out[2] = -1; out[3] = 1;
    }
  }
  if (lane == 0) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<i32x4*>(a.runs + 4 * t) = i32x4{out[0], out[1], out[2], out[3]};
  }
}

}  // namespace

hipError_t launch_swa_runs(const SwaRunsArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int64_t grid = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL(swa_runs_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
