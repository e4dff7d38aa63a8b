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
// Each wave owns 64 consecutive output rows (four waves per 256-thread workgroup). Per row, bf16:
// lane l copies bytes 16 l .. 16 l + 15 of the first 1 KB, lanes 0..7 the last 128 bytes (d_qk 576);
// fp8: lane l < d_nope / 8 widens eight codes of group l / 8 with v_cvt_scalef32_pk_bf16_fp8 into
// 16 bytes, lanes 0..7 copy the RoPE tail. Loads and stores are contiguous per row.
#include "layer_internal.h"

namespace mla {

namespace {

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

// Source of one output row: its row's bytes and (fp8) its scale slot, or 0 for a zero row.
template <bool FP8, int DQK>
__device__ __forceinline__ void row_source(const GatherArgs& a, int64_t i, uint64_t* row, uint64_t* sc) {
  constexpr int kNope = DQK - 64;
  *row = 0;
  *sc = 0;
  if (i >= a.n) return;
  const int r = a.token_to_seq[i];
  const int64_t j = (a.seq_starts != nullptr ? (int64_t)a.seq_starts[r] : 0) + i - a.cu_seq_lens[r];
  if (j < 0 || (j >> a.ps_log2) >= a.max_pages) return;
  const int64_t page = a.block_table[(int64_t)r * a.max_pages + (j >> a.ps_log2)];
  if (page < 0 || page >= a.num_pages) return;
  const int slot = (int)(j & ((1 << a.ps_log2) - 1));
  const uint8_t* pg = a.cache + page * a.page_stride;
  *row = (uint64_t)(uintptr_t)(pg + (int64_t)slot * (FP8 ? kNope + 128 : 2 * DQK));
  *sc = (uint64_t)(uintptr_t)(pg + a.scale_off + 8 * slot);
}

__device__ __forceinline__ uint64_t lane64(uint64_t v, int k) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, k);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), k);
  return ((uint64_t)hi << 32) | lo;
}

// Wave w of the grid takes output rows 64 w .. 64 w + 63: lane l resolves row 64 w + l (request,
// position, page: three dependent loads, paid once per 64 rows), then the wave copies the rows four
// at a time, all four rows' loads issued before their stores.
template <bool FP8, int DQK>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int kNope = DQK - 64;
  const int lane = threadIdx.x & 63;
  const int64_t i0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  if (i0 >= a.n) return;
  uint64_t my_row, my_sc;
  row_source<FP8, DQK>(a, i0 + lane, &my_row, &my_sc);
  const int rows = (int)min((int64_t)64, a.n - i0);
  for (int k0 = 0; k0 < rows; k0 += 4) {
    u32x4 v[4], pe[4];
    u32x2 codes[4];
    float scale[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = min(k0 + q, rows - 1);
      const uint8_t* src = reinterpret_cast<const uint8_t*>((uintptr_t)lane64(my_row, k));
      const uint8_t* sc = reinterpret_cast<const uint8_t*>((uintptr_t)lane64(my_sc, k));
      v[q] = u32x4{0u, 0u, 0u, 0u};
      pe[q] = u32x4{0u, 0u, 0u, 0u};
      codes[q] = u32x2{0u, 0u};
      scale[q] = 0.f;
      if (src != nullptr) {
        if constexpr (!FP8) {
          v[q] = *reinterpret_cast<const u32x4*>(src + 16 * lane);
          if (DQK > 512 && lane < 8) pe[q] = *reinterpret_cast<const u32x4*>(src + 1024 + 16 * lane);
        } else {
          if (lane < kNope / 8) {
            codes[q] = *reinterpret_cast<const u32x2*>(src + 8 * lane);
            scale[q] = ue8m0_scale(sc[lane >> 3]);
          }
          if (lane < 8) pe[q] = *reinterpret_cast<const u32x4*>(src + kNope + 16 * lane);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (k0 + q >= rows) break;
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.dst) + (i0 + k0 + q) * (2 * DQK);
      if constexpr (!FP8) {
        *reinterpret_cast<u32x4*>(dst + 16 * lane) = v[q];
        if (DQK > 512 && lane < 8) *reinterpret_cast<u32x4*>(dst + 1024 + 16 * lane) = pe[q];
      } else {
        if (lane < kNope / 8) *reinterpret_cast<u32x4*>(dst + 16 * lane) = widen8(codes[q], scale[q]);
        if (lane < 8) *reinterpret_cast<u32x4*>(dst + 2 * kNope + 16 * lane) = pe[q];
      }
    }
  }
}

template <bool FP8, int DQK>
hipError_t launch_t(const GatherArgs& a, hipStream_t s) {
  const int64_t grid = (a.n + 4 * 64 - 1) / (4 * 64);
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
