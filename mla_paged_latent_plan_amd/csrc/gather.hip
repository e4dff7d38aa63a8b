// mla_gather_context kernel: context rows gathered from the paged cache into a contiguous bf16
// workspace (vLLM mla_attention.py, _compute_prefill_context: gather_and_maybe_dequant_cache
// with cu_seq_lens, token_to_seq and seq_starts), so that the chunked-context prefill can
// up-project them.
//
// Output row i belongs to request r = token_to_seq[i] and holds that request's logical row
// j = seq_starts[r] + i - cu_seq_lens[r], read from page block_table[r, j / page_size], slot
// j % page_size. bf16 rows are copied; fp8 rows are widened: value = e4m3(code) * 2^(e - 127) for
// the ue8m0 byte e of its 64-value group (exact in bf16), the RoPE tail copied as bf16. Rows whose
// position or page lies outside the cache are written as zeros.
//
// One wave per output row, four rows per 256-thread workgroup. bf16 rows: lane l copies bytes
// 16 l .. 16 l + 15 of the first 1 KB, lanes 0..7 the last 128 bytes (d_qk 576). fp8 rows: lane
// l < d_nope / 8 widens eight codes of group l / 8 with v_cvt_scalef32_pk_bf16_fp8 into 16 bytes,
// lanes 0..7 copy the RoPE tail. Loads and stores are contiguous per row.
#include "layer_internal.h"

namespace mla {

namespace {

constexpr int kRowsPerBlock = 4;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ue8m0_scale(uint32_t s) {
  const uint32_t bits = (s == 0u) ? 0x00400000u : ((s == 255u) ? 0x7FC00000u : (s << 23));
  return __uint_as_float(bits);
}

__device__ __forceinline__ u32x4 widen8(u32x2 codes, float sc) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], sc, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], sc, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], sc, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], sc, true);
  return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
               __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

template <bool FP8, int DQK>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int kNope = DQK - 64;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (i >= a.n) return;
  const int r = a.token_to_seq[i];
  const int64_t j = (a.seq_starts != nullptr ? (int64_t)a.seq_starts[r] : 0) + i - a.cu_seq_lens[r];
  int64_t page = -1;
  if (j >= 0 && (j >> a.ps_log2) < a.max_pages) page = a.block_table[(int64_t)r * a.max_pages + (j >> a.ps_log2)];
  uint8_t* dst = reinterpret_cast<uint8_t*>(a.dst) + i * (2 * DQK);
  if (page < 0 || page >= a.num_pages) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = z;
    if (DQK > 512 && lane < 8) *reinterpret_cast<u32x4*>(dst + 1024 + 16 * lane) = z;
    return;
  }
  const int slot = (int)(j & ((1 << a.ps_log2) - 1));
  const uint8_t* pg = a.cache + page * a.page_stride;
  if constexpr (!FP8) {
    const uint8_t* src = pg + (int64_t)slot * (2 * DQK);
    *reinterpret_cast<u32x4*>(dst + 16 * lane) = *reinterpret_cast<const u32x4*>(src + 16 * lane);
    if (DQK > 512 && lane < 8)
      *reinterpret_cast<u32x4*>(dst + 1024 + 16 * lane) = *reinterpret_cast<const u32x4*>(src + 1024 + 16 * lane);
  } else {
    const uint8_t* src = pg + (int64_t)slot * (kNope + 128);
    const uint8_t* scales = pg + a.scale_off + 8 * slot;
    // lanes < kNope / 8 widen eight codes each; lanes 0..7 also copy the RoPE tail (128 bytes)
    if (lane < kNope / 8) {
      const u32x2 codes = *reinterpret_cast<const u32x2*>(src + 8 * lane);
      const float sc = ue8m0_scale(scales[lane >> 3]);
      *reinterpret_cast<u32x4*>(dst + 16 * lane) = widen8(codes, sc);
    }
    if (lane < 8)
      *reinterpret_cast<u32x4*>(dst + 2 * kNope + 16 * lane) = *reinterpret_cast<const u32x4*>(src + kNope + 16 * lane);
  }
}

template <bool FP8, int DQK>
hipError_t launch_t(const GatherArgs& a, hipStream_t s) {
  const int64_t grid = (a.n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((gather_kernel<FP8, DQK>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int fmt, int d_qk, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (fmt == 0) return d_qk == 576 ? launch_t<false, 576>(a, s) : launch_t<false, 512>(a, s);
  return d_qk == 576 ? launch_t<true, 576>(a, s) : launch_t<true, 512>(a, s);
}

}  // namespace mla
