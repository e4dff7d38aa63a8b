// Internal definitions of the kernels around the decode (absorption GEMMs, sliding-window run
// plan, context gather, sparse prefill metadata) shared with the C-ABI layer.
#pragma once

#include "mla_internal.h"

namespace mla {

// Per-head NT GEMM C[t, h, n] = sum_k A[t, h, k] W[h, n, k] (bf16 in/out, fp32 accumulation),
// optionally followed by a copy of pe[t, h, 0:R] into C[t, h, N:N+R]. Strides in elements.
struct GemmArgs {
  const uint16_t* a;
  int64_t a_t, a_h;
  const uint16_t* w;  // [H][N][K]
  uint16_t* c;
  int64_t c_t, c_h;
  const uint16_t* pe;  // nullable
  int64_t pe_t, pe_h;
  int T, H, N, K, R;
};

struct SwaRunsArgs {
  const int32_t* kv;       // [T][topk] window slots
  const int32_t* lengths;  // [T] or nullptr
  int32_t* runs;           // [T][4]
  int64_t T;
  int topk, ps_log2, step;
};

struct GatherArgs {
  const uint8_t* cache;
  const int32_t* block_table;   // [num_reqs][max_pages]
  const int32_t* cu_seq_lens;   // [num_reqs + 1]
  const int32_t* seq_starts;    // [num_reqs] or nullptr
  const int32_t* token_to_seq;  // [n]
  uint16_t* dst;                // bf16 [n][d_qk]
  int64_t n, page_stride, num_pages, scale_off;
  int max_pages, ps_log2;
};

hipError_t launch_absorb_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, int fmt, int d_qk, hipStream_t s);
hipError_t launch_swa_runs(const SwaRunsArgs& a, hipStream_t s);
// meta[0] = s_kv, meta[1 + i] = i for i < pages (pages >= 1).
hipError_t launch_sparse_meta(int32_t* meta, int32_t s_kv, int32_t pages, hipStream_t s);

}  // namespace mla
