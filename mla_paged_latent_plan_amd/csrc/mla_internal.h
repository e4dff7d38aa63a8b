// Internal definitions shared by the plan, decode, combine and cache-write kernels and the C-ABI
// layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// ---- plan layout (int32 words) -------------------------------------------------------------
// header[16] | grp_ptr[G+1] | unit_ptr[U+1] | grp_rows[2G] | splits[4*(G+U)] | pad to 256 B |
// zero rows (kZeroRowBytes) | split descriptors [G+U][8]: (g, b, j0, n, L, q0, qend, nsplit) of
// each split, everything a decode kernel needs to start it, in one 32-byte record
constexpr int32_t kPlanMagic = 0x4D4C4131;
constexpr int kHeaderWords = 16;
constexpr int kBlockRows = 64;       // rows per block (one LDS stage)
// Zero rows: eight of the widest row (1152 B), rounded up. The 128-row tile addresses row i of an
// eight-row run as page base + i * row bytes (+ an offset inside the row), and an out-of-range
// page entry gives the zero row as that base, so reads reach up to 8 rows past it.
constexpr int kZeroRowBytes = 9472;
constexpr int kMaxGroups = 8192;     // plan kernel keeps per-group state in LDS
constexpr int kDv = 512;

enum { H_MAGIC = 0, H_G, H_U, H_S, H_R, H_MTILES, H_MTILE, H_QUOTA, H_FIXED, H_TOTAL, H_SMAX };

struct PlanLayout {
  int64_t G, U;
  int64_t grp_ptr, unit_ptr, grp_rows, splits, words;  // word offsets
  int64_t zero_row_bytes_off, sdesc_bytes_off, bytes;   // byte offsets / size
  static PlanLayout make(int64_t G, int64_t U) {
    PlanLayout l;
    l.G = G;
    l.U = U;
    l.grp_ptr = kHeaderWords;
    l.unit_ptr = l.grp_ptr + G + 1;
    l.grp_rows = l.unit_ptr + U + 1;
    l.splits = l.grp_rows + 2 * G;
    l.words = l.splits + 4 * (G + U);
    l.zero_row_bytes_off = ((l.words * 4 + 255) / 256) * 256;
    l.sdesc_bytes_off = l.zero_row_bytes_off + kZeroRowBytes;
    l.bytes = l.sdesc_bytes_off + 32 * (G + U);
    return l;
  }
};

// Kernel tile for R stacked query rows per group: (M_TILE, FIXED split overhead in blocks).
inline void tile_params(int R, int* m_tile, int* fixed) {
  if (R <= 16) { *m_tile = 16; *fixed = 3; }
  else if (R <= 32) { *m_tile = 32; *fixed = 2; }
  else if (R <= 64) { *m_tile = 64; *fixed = 4; }
  else { *m_tile = 128; *fixed = 4; }
}

struct Shape {  // derived, validated problem shape
  int B, Sq, H, R, G, m_tile, fixed, m_tiles, U, d_qk, d_rope, fmt, page_size, ps_log2;
  int max_pages, topk, causal, window;
  int64_t page_stride, num_pages, row_bytes, s_max;
};

// ---- kernel argument blocks ----------------------------------------------------------------
struct PlanArgs {
  const int32_t* seqlens;
  const int32_t* topk_lens;
  int32_t* plan;
  PlanLayout lay;
  int B, Sq, R, G, U, m_tiles, m_tile, fixed, topk, window;
};

struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* cache;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;
  const float* sink;
  const int32_t* plan;
  const uint8_t* zero_row;
  uint16_t* part_o;  // bf16 [S_max][R][512] partial outputs, each normalised by its own sum
  float* part_lse;
  uint16_t* out;
  float* lse;
  float* max_logits;  // optional: per-row maximum scaled score (LSE layout), or nullptr
  float* part_max;    // fp32 [S_max][R] per-split maxima; used only with max_logits
  int64_t page_stride, num_pages, row_bytes;
  int64_t scale_off;  // fp8 rows: byte offset of a page's scale slots (page_size * row_bytes)
  int64_t grp_ptr_off, unit_ptr_off, grp_rows_off, splits_off, sdesc_off;
  int B, Sq, H, R, G, U, m_tiles, ps_log2, max_pages, topk, causal, window;
  float scale_log2;  // sm_scale * log2(e)
};

struct CombineArgs {
  const int32_t* plan;
  const uint16_t* part_o;
  const float* part_lse;
  const float* sink;
  uint16_t* out;
  float* lse;
  const float* part_max;  // with max_logits: per-split maxima written by the decode
  float* max_logits;      // optional, or nullptr
  int64_t grp_ptr_off;
  int B, Sq, H, R, G, U;
  int sparse;
};

// Whether a plan's header describes the problem a kernel was launched for (magic word, groups,
// units, stacked rows per group, partial slots): a plan built for another problem or CU count is
// not used.
__device__ __forceinline__ bool plan_matches(const int32_t* plan, int G, int U, int R) {
  const int magic = __builtin_amdgcn_readfirstlane(plan[H_MAGIC]);
  const int g = __builtin_amdgcn_readfirstlane(plan[H_G]);
  const int u = __builtin_amdgcn_readfirstlane(plan[H_U]);
  const int r = __builtin_amdgcn_readfirstlane(plan[H_R]);
  const int smax = __builtin_amdgcn_readfirstlane(plan[H_SMAX]);
  return magic == kPlanMagic && g == G && u == U && r == R && smax == G + U;
}

// The split range [s0, s1) of a decode work unit, requested with the plan's header words (one
// memory round trip for both); false when the unit is past U or the plan is of another problem.
// (Without EARLY, the range is read after the test: kernels whose scalar registers are short keep
// the two words out of the header's round trip.)
template <bool EARLY = true>
__device__ __forceinline__ bool unit_splits(const DecodeArgs& a, int unit, int* s0, int* s1) {
  if constexpr (EARLY) {
    const int uc = min(unit, a.U - 1);
    const int b0 = a.plan[a.unit_ptr_off + uc];
    const int b1 = a.plan[a.unit_ptr_off + uc + 1];
    const bool match = plan_matches(a.plan, a.G, a.U, a.R);
    asm volatile("" ::"s"(b0), "s"(b1));  // issued before the test
    *s0 = b0;
    *s1 = b1;
    return match && unit < a.U;
  } else {
    if (unit >= a.U || !plan_matches(a.plan, a.G, a.U, a.R)) return false;
    *s0 = a.plan[a.unit_ptr_off + unit];
    *s1 = a.plan[a.unit_ptr_off + unit + 1];
    return true;
  }
}

struct KvWriteArgs {
  const uint16_t* kv_c;  // bf16 [n][d_nope]
  const uint16_t* k_pe;  // bf16 [n][64]
  const int64_t* slots;  // [n]
  uint8_t* cache;
  int64_t n, num_slots, page_stride;
  int64_t scale_off;  // fp8 rows: byte offset of a page's scale slots (page_size * row_bytes)
  int ps_log2;
};

// Checked mode: the inputs of a decode call tested against the contract (csrc/check.hip).
struct CheckArgs {
  const int32_t* plan;
  const int32_t* block_table;
  const int32_t* seqlens;
  const int32_t* indices;  // index lists, or nullptr
  int64_t num_pages;
  int64_t grp_rows_off;    // plan words: (first row, row count) per group
  int B, Sq, R, G, U, ps_log2, max_pages, topk, window;
};

// Launchers (defined in the .hip files).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, const Shape& sh, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_kv_write(const KvWriteArgs& a, int fmt, int d_nope, hipStream_t s);
hipError_t launch_check(const CheckArgs& a, hipStream_t s);
// The current device's checked-mode bits (after the stream's work), cleared on request.
hipError_t check_status(uint32_t* bits, bool clear, hipStream_t s);

}  // namespace mla
