// Checked mode: a decode call's inputs tested against the contract the decode kernels assume,
// with violations recorded as bits of a per-device word instead of being read silently as zero
// rows. The decode kernels themselves stay unchecked; this kernel runs before them on the stream.
//   MLA_CHECK_PAGE    a block-table entry outside [0, num_pages) for a page holding a visible row
//                     (dense: the request's rows, or the window's; index lists: a listed row in
//                     [0, L))
//   MLA_CHECK_LENGTH  a visible row past the block table (page index >= max_pages_per_seq)
//   MLA_CHECK_PLAN    a plan whose header does not describe this problem and CU count
#include "mla_internal.h"

namespace mla {

__device__ __align__(16) uint32_t check_word[4];  // [0]: violation bits since the last clear

namespace {

__device__ __forceinline__ void flag(uint32_t bits) {
  if (bits != 0) atomicOr(&check_word[0], bits);
}

__global__ __launch_bounds__(256) void check_kernel(CheckArgs a) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  const int32_t* h = a.plan;
  const bool plan_ok = h[H_MAGIC] == kPlanMagic && h[H_G] == a.G && h[H_U] == a.U && h[H_R] == a.R &&
                       h[H_SMAX] == a.G + a.U;
  if (tid == 0) flag(plan_ok ? 0u : 4u);
  const int ps = 1 << a.ps_log2;
  uint32_t bits = 0;
  if (a.topk == 0) {
    // every (request, page) pair of the block table
    const int64_t n = (int64_t)a.B * a.max_pages;
    for (int64_t x = tid; x < n; x += nthreads) {
      const int b = (int)(x / a.max_pages), i = (int)(x % a.max_pages);
      const int L = a.seqlens[b];
      if (L <= 0) continue;
      const int j0 = (a.window > 0) ? max(0, L - (a.window + a.Sq - 1)) : 0;
      const int64_t lo = (int64_t)i * ps, hi = lo + ps;  // rows of page i: [lo, hi)
      if (hi <= j0 || lo >= L) continue;
      const int page = a.block_table[x];
      if (page < 0 || (int64_t)page >= a.num_pages) bits |= 1u;
      if (i == a.max_pages - 1 && (int64_t)L > hi) bits |= 2u;  // rows past the last page
    }
  } else if (plan_ok) {
    // every index entry of every (request, token) within the token's row count (from the plan)
    const int64_t n = (int64_t)a.B * a.Sq * a.topk;
    for (int64_t x = tid; x < n; x += nthreads) {
      const int64_t g = x / a.topk;
      const int k = (int)(x % a.topk);
      const int b = (int)(g / a.Sq);
      const int L = a.seqlens[b];
      if (L <= 0) continue;
      const int len = a.plan[a.grp_rows_off + 2 * g + 1];
      if (k >= len) continue;
      const int j = a.indices[x];
      if (j < 0 || j >= L) continue;  // skipped entries, part of the contract
      const int pi = j >> a.ps_log2;
      if (pi >= a.max_pages) {
        bits |= 2u;
        continue;
      }
      const int page = a.block_table[(int64_t)b * a.max_pages + pi];
      if (page < 0 || (int64_t)page >= a.num_pages) bits |= 1u;
    }
  }
  flag(bits);
}

}  // namespace

// The word's device address is taken per call with hipGetSymbolAddress (in host code the name
// `check_word` is a host-side stand-in), then read, and cleared, with plain synchronous copies.
hipError_t check_status(uint32_t* bits, bool clear, hipStream_t s) {
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(check_word));
  if (e != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  if ((e = hipMemcpy(bits, ptr, sizeof(uint32_t), hipMemcpyDeviceToHost)) != hipSuccess) return e;
  if (clear) {
    const uint32_t zero = 0;
    e = hipMemcpy(ptr, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
  }
  return e;
}

hipError_t launch_check(const CheckArgs& a, hipStream_t s) {
  const int64_t n = (a.topk == 0) ? (int64_t)a.B * a.max_pages : (int64_t)a.B * a.Sq * a.topk;
  const int64_t blocks = max((int64_t)1, min((int64_t)1024, (n + 255) / 256));
  hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
