// mla_kv_write kernel: new tokens' latent rows written in place into the paged cache (vLLM
// mla_attention.py, update_kv_cache(kv_c_normed, k_pe, kv_cache, slot_mapping, ...); HALOps MLA
// API, mla_attention kv_cache: each token's new row is written in place).
//
// Token i's row goes to slot s = slot_mapping[i]: physical page s >> log2(page_size), row
// s & (page_size - 1). bf16 rows are [kv_c | k_pe] copied as they are. fp8 rows (HALOps kv_cache
// layout) are [e4m3fn codes of kv_c | k_pe as bf16], and the page's scale slot of the row holds one
// ue8m0 byte per 64 kv_c values (zero pad bytes). A group's scale is 2^k for the smallest integer k
// with amax <= 448 * 2^k (clamped to [-127, 127]; an all-zero group gets k = 0), and each code is
// value * 2^-k rounded to the nearest e4m3fn value, ties to even: |value * 2^-k| <= 448, so the
// conversion never saturates.
//
// Launch: 256-thread workgroups, at most 32 waves per compute unit, each wave taking a contiguous
// run of tokens one at a time, with the next token's row loaded ahead. Each lane owns eight
// consecutive kv_c values (16 bytes in, 8 fp8 bytes out), so the eight lanes of a 64-value group
// find its maximum with three butterfly steps; the RoPE tail is 8 lanes x 16 bytes. Loads and
// stores are contiguous per row. HBM-bound: per token 2 * d_qk bytes in and the row (+ 8-byte scale
// slot) out.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTokensPerBlock = 4;  // one wave per token
constexpr int kWavesPerCu = 32;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// e4m3fn code of y (|y| <= 448), round to nearest even. The hardware conversion is used where y is
// at least the smallest fp32 normal; below 2^-10 (half the smallest e4m3 subnormal, a tie that goes
// to the even code 0) the code is the signed zero, set explicitly so that fp32 denormal handling
// cannot change the sign.
__device__ __forceinline__ uint32_t fp8_pair(float y0, float y1) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  uint32_t c0 = (uint32_t)w & 0xFFu, c1 = ((uint32_t)w >> 8) & 0xFFu;
  if (fabsf(y0) <= 0x1p-10f) c0 = (__float_as_uint(y0) >> 24) & 0x80u;
  if (fabsf(y1) <= 0x1p-10f) c1 = (__float_as_uint(y1) >> 24) & 0x80u;
  return c0 | (c1 << 8);
}

// k of the scale 2^k: smallest integer with amax <= 448 * 2^k (448 = 0.875 * 2^9), clamped.
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e = 0;
  const float m = frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
  const int k = (m <= 0.875f) ? e - 9 : e - 8;
  return min(127, max(-127, k));
}

// One token's source data in registers: lane's 16 bytes of kv_c (lanes < DNOPE / 8) and of k_pe
// (lanes < 8), and the token's slot.
struct Src {
  u32x4 c, p;
  int64_t slot;
};

template <int DNOPE>
__device__ __forceinline__ Src load_src(const KvWriteArgs& a, int64_t i, int lane) {
  Src s;
  s.c = u32x4{0u, 0u, 0u, 0u};
  s.p = u32x4{0u, 0u, 0u, 0u};
  s.slot = -1;
  if (i < a.n) {
    s.slot = a.slots[i];
    const uint8_t* src_c = reinterpret_cast<const uint8_t*>(a.kv_c) + i * (2 * DNOPE);
    const uint8_t* src_p = reinterpret_cast<const uint8_t*>(a.k_pe) + i * 128;
    if (lane < DNOPE / 8) s.c = *reinterpret_cast<const u32x4*>(src_c + 16 * lane);
    if (lane < 8) s.p = *reinterpret_cast<const u32x4*>(src_p + 16 * lane);
  }
  return s;
}

// bf16 rows: [kv_c | k_pe] stored as given, 16 bytes per lane.
template <int DNOPE>
__device__ __forceinline__ void store_bf16(const KvWriteArgs& a, const Src& s, int lane) {
  const int64_t page = s.slot >> a.ps_log2;
  const int r = (int)(s.slot & ((1 << a.ps_log2) - 1));
  uint8_t* dst = a.cache + page * a.page_stride + (int64_t)r * (2 * DNOPE + 128);
  if (lane < DNOPE / 8) *reinterpret_cast<u32x4*>(dst + 16 * lane) = s.c;
  if (lane < 8) *reinterpret_cast<u32x4*>(dst + 2 * DNOPE + 16 * lane) = s.p;
}

// fp8 rows: codes of kv_c, k_pe as bf16, and the row's scale slot.
template <int DNOPE>
__device__ __forceinline__ void store_fp8(const KvWriteArgs& a, const Src& s, int lane) {
  constexpr int kGroups = DNOPE / 64;
  const int64_t page = s.slot >> a.ps_log2;
  const int r = (int)(s.slot & ((1 << a.ps_log2) - 1));
  uint8_t* pg = a.cache + page * a.page_stride;
  uint8_t* dst = pg + (int64_t)r * (DNOPE + 128);
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(s.c[j]);
    v[2 * j + 1] = bf16_hi(s.c[j]);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  // the group's eight lanes are lanes 8g .. 8g + 7
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  const int k = scale_exp(amax);
  u32x2 codes;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t lo = fp8_pair(ldexpf(v[4 * j], -k), ldexpf(v[4 * j + 1], -k));
    const uint32_t hi = fp8_pair(ldexpf(v[4 * j + 2], -k), ldexpf(v[4 * j + 3], -k));
    codes[j] = lo | (hi << 16);
  }
  if (lane < 8 * kGroups) *reinterpret_cast<u32x2*>(dst + 8 * lane) = codes;
  if (lane < 8) *reinterpret_cast<u32x4*>(dst + DNOPE + 16 * lane) = s.p;
  // scale slot: byte g = 127 + k of group g (lane 8g), pad bytes zero
  uint32_t sb[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) sb[g] = (g < kGroups) ? (uint32_t)(127 + __shfl(k, 8 * g, 64)) : 0u;
  if (lane == 0) {
    const u32x2 w = {sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24),
                     sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24)};
    *reinterpret_cast<u32x2*>(pg + a.scale_off + 8 * r) = w;
  }
}

// Wave w takes the contiguous run of tokens [w C, w C + C), C = ceil(n / W) for W waves in the
// grid: tokens written in slot order (a prefill) then fill a page's rows and its shared scale-slot
// lines from one compute unit, whose L2 merges the 8-byte slot writes into whole lines. The next
// token's loads are issued before the current token is converted and stored.
template <bool FP8, int DNOPE>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t C = (a.n + W - 1) / W;
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  int64_t i = w * C;
  const int64_t end = (i + C < a.n) ? i + C : a.n;
  Src cur = load_src<DNOPE>(a, i < end ? i : a.n, lane);
  for (; i < end; ++i) {
    const Src nxt = load_src<DNOPE>(a, i + 1 < end ? i + 1 : a.n, lane);
    // no slot, or a slot outside the cache: skipped (wave-uniform)
    if (cur.slot >= 0 && cur.slot < a.num_slots) {
      if constexpr (FP8) store_fp8<DNOPE>(a, cur, lane);
      else store_bf16<DNOPE>(a, cur, lane);
    }
    cur = nxt;
  }
}

template <bool FP8, int DNOPE>
hipError_t launch_t(const KvWriteArgs& a, hipStream_t s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  // up to kWavesPerCu waves per compute unit, none without a token
  const int64_t waves = (a.n < (int64_t)cus * kWavesPerCu) ? a.n : (int64_t)cus * kWavesPerCu;
  const int64_t grid = (waves + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL((kv_write_kernel<FP8, DNOPE>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs& a, int fmt, int d_nope, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (fmt == 0) return d_nope == 512 ? launch_t<false, 512>(a, s) : launch_t<false, 448>(a, s);
  return d_nope == 512 ? launch_t<true, 512>(a, s) : launch_t<true, 448>(a, s);
}

}  // namespace mla
