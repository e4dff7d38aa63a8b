// mla_combine kernel: log-sum-exp merge of split partials (vLLM merge_attn_states; HALOps
// mla_output_proj, "split-KV LSE combine"), then the attention sink.
//
// For each query group whose split count is not one: LSE = ln sum_i exp(LSE_i) and
// O = sum_i exp(LSE_i - LSE) O_i over the group's splits; a split with no visible rows carries
// LSE_i = -inf and no weight (vLLM neutralize_empty_context_partials). The sink (HALOps attn_sink)
// then adds exp(sink_h) once to the denominator. A group with no splits at all gets O = 0 and
// LSE = -inf, or LSE = sink_h with a sink. Groups with exactly one split were finished by
// mla_decode and are skipped. On request the row's largest scaled score is the largest of its
// splits' (-inf without splits).
//
// Launch: workgroups of 256 threads over (4 query rows, group); 64 threads per row, each owning 8
// consecutive columns, so bf16 partial rows are read as contiguous 1 KB lines. Lane i reads the LSE
// of split i (per chunk of 64 splits); seven splits' rows are loaded before they are accumulated,
// through buffer loads (a scalar descriptor per split block, one lane offset for all), and at most
// 64 VGPRs keep eight waves on each SIMD, so a grid of 2048 workgroups is resident at once.
// Groups with more than one split number at most U - 1 (each straddles a unit boundary), so the
// grid's group dimension is capped at U and a workgroup strides over groups; those with one split
// (already final) cost it only their two split pointers.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kDepth = 7;  // partial rows in flight per lane (groups of three or more splits)
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void combine_group(const CombineArgs& a, int g, int s0, int s1);

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
void combine_kernel(CombineArgs a) {
  // The split pointers of the workgroup's first four groups are requested with the plan's header
  // words, one memory round trip for both; they are used only if the header matches.
  const int gstep = gridDim.y;
  int p0[4], p1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = min((int)blockIdx.y + i * gstep, a.G - 1);
    p0[i] = a.plan[a.grp_ptr_off + g];
    p1[i] = a.plan[a.grp_ptr_off + g + 1];
  }
  const bool match = plan_matches(a.plan, a.G, a.U, a.R);
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" ::"s"(p0[i]), "s"(p1[i]));  // issued before the test
  if (!match) {
#pragma unroll 1
    // a plan of another problem: the decode skipped its work, and every output row is NaN
    for (int g = blockIdx.y; g < a.G; g += gridDim.y) {
      const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
      if (r >= a.R) continue;
      const int lane = threadIdx.x & 63;
      const uint4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
      *reinterpret_cast<uint4*>(a.out + ((int64_t)g * a.R + r) * kDv + 8 * lane) = nan4;
      if (lane == 0) {
        const int b = a.sparse ? g / a.Sq : g, t = a.sparse ? g % a.Sq : r / a.H, h = a.sparse ? r : r % a.H;
        a.lse[((int64_t)b * a.H + h) * a.Sq + t] = __builtin_nanf("");
        if (a.max_logits != nullptr) a.max_logits[((int64_t)b * a.H + h) * a.Sq + t] = __builtin_nanf("");
      }
    }
    return;
  }
  // a workgroup whose groups all have one split (finished by the decode) leaves at once
  bool work = (int)blockIdx.y + 4 * gstep < a.G;
#pragma unroll
  for (int i = 0; i < 4; ++i) work |= ((int)blockIdx.y + i * gstep < a.G) && (p1[i] - p0[i] != 1);
  if (!work) return;
#pragma unroll 1
  for (int i = 0, g = (int)blockIdx.y; g < a.G; ++i, g += gstep) {
    int s0, s1;
    if (i < 4) {
      s0 = (i == 0) ? p0[0] : (i == 1) ? p0[1] : (i == 2) ? p0[2] : p0[3];
      s1 = (i == 0) ? p1[0] : (i == 1) ? p1[1] : (i == 2) ? p1[2] : p1[3];
    } else {
      s0 = a.plan[a.grp_ptr_off + g];
      s1 = a.plan[a.grp_ptr_off + g + 1];
    }
    s0 = __builtin_amdgcn_readfirstlane(s0);
    s1 = __builtin_amdgcn_readfirstlane(s1);
    if (s1 - s0 != 1) combine_group(a, g, s0, s1);
  }
}

// The merge of group g's splits [s0, s1) for the workgroup's four rows.
__device__ __forceinline__ void combine_group(const CombineArgs& a, int g, int s0, int s1) {
  constexpr int D = kDepth;
  const int ns = s1 - s0;
  const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= a.R) return;
  const int lane = threadIdx.x & 63;
  const int c = lane * 8;

  int b, t, h;
  if (a.sparse) {
    b = g / a.Sq;
    t = g % a.Sq;
    h = r;
  } else {
    b = g;
    t = r / a.H;
    h = r % a.H;
  }

  // The row's split weights: lane i holds split s0 + i of each 64-split chunk. The first chunk's
  // LSEs and the first D splits' rows are requested together, so a group with at most D splits
  // costs one memory round trip before its sums; larger groups then load D rows at a
  // time. Rows are accumulated in split order.
  // A split's partial block is R rows of 1 KB: the row's columns sit at a lane offset below 2^32
  // bytes in each block, and the block's address is wave-uniform (a scalar base plus that offset).
  const uint32_t lane_off = (uint32_t)(r * kDv + c) * 2u;
  const uint8_t* pbase = reinterpret_cast<const uint8_t*>(a.part_o) + (int64_t)s0 * a.R * kDv * 2;
  const int64_t pstep = (int64_t)a.R * kDv * 2;
  // buffer load of split block i: a scalar descriptor and the lane offset
  auto ld = [&](int i) -> uint4 {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(pbase + i * pstep), (short)0, (int)pstep, 0x00020000);
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, 0, 0);
    return uint4{w[0], w[1], w[2], w[3]};
  };

  // (indices past the group's last split repeat it: loads whose rows are not accumulated; groups
  // of two splits, from short windows or index lists of a few blocks, skip the other five)
  uint4 v[D];
  if (ns > 0) {
    v[0] = ld(0);
    v[1] = ld(min(1, ns - 1));
    if (ns > 2) {
#pragma unroll
      for (int q = 2; q < D; ++q) v[q] = ld(min(q, ns - 1));
    }
  }
  float ls0 = (lane < ns) ? a.part_lse[(int64_t)(s0 + lane) * a.R + r] : kNegInf;
  float mx = ls0;
  for (int s = s0 + 64; s < s1; s += 64)
    if (s + lane < s1) mx = fmaxf(mx, a.part_lse[(int64_t)(s + lane) * a.R + r]);
  mx = wave_max(mx);
  float wsum = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (mx != kNegInf) {
    for (int sc = s0; sc < s1; sc += 64) {
      const float ls = (sc == s0) ? ls0
                                  : (sc + lane < s1) ? a.part_lse[(int64_t)(sc + lane) * a.R + r] : kNegInf;
      const float wl = (ls == kNegInf) ? 0.f : __expf(ls - mx);
      wsum += wl;
      const int nc = min(64, s1 - sc);
      for (int k = 0; k < nc; k += D) {
        if (sc != s0 || k != 0) {  // the first D rows are already loaded
#pragma unroll
          for (int q = 0; q < D; ++q)
            v[q] = ld(sc - s0 + min(k + q, nc - 1));
        }
#pragma unroll
        for (int q = 0; q < D; ++q) {
          if (k + q < nc) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k + q));
            const uint32_t u[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[2 * i] += w * __uint_as_float(u[i] << 16);
              acc[2 * i + 1] += w * __uint_as_float(u[i] & 0xFFFF0000u);
            }
          }
        }
      }
    }
    wsum = wave_sum(wsum);
  }
  float lse, scale;
  if (wsum > 0.f) {
    lse = mx + __logf(wsum);
    scale = 1.f / wsum;
  } else {
    lse = kNegInf;
    scale = 0.f;
  }
  if (a.sink != nullptr) {
    const float sk = a.sink[h];
    if (lse == kNegInf) {
      lse = sk;
      scale = 0.f;
    } else {
      const float m2 = fmaxf(lse, sk);
      const float lse2 = m2 + __logf(__expf(lse - m2) + __expf(sk - m2));
      scale *= __expf(lse - lse2);
      lse = lse2;
    }
  }
  uint4 w;
  w.x = (uint32_t)f2bf(acc[0] * scale) | ((uint32_t)f2bf(acc[1] * scale) << 16);
  w.y = (uint32_t)f2bf(acc[2] * scale) | ((uint32_t)f2bf(acc[3] * scale) << 16);
  w.z = (uint32_t)f2bf(acc[4] * scale) | ((uint32_t)f2bf(acc[5] * scale) << 16);
  w.w = (uint32_t)f2bf(acc[6] * scale) | ((uint32_t)f2bf(acc[7] * scale) << 16);
  *reinterpret_cast<uint4*>(a.out + ((int64_t)g * a.R + r) * kDv + c) = w;
  if (lane == 0) a.lse[((int64_t)b * a.H + h) * a.Sq + t] = lse;
  if (a.max_logits != nullptr) {
    float pm = kNegInf;
    for (int s = s0; s < s1; s += 64)
      if (s + lane < s1) pm = fmaxf(pm, a.part_max[(int64_t)(s + lane) * a.R + r]);
    pm = wave_max(pm);
    if (lane == 0) a.max_logits[((int64_t)b * a.H + h) * a.Sq + t] = pm;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.G <= 0) return hipSuccess;
  dim3 grid((a.R + kRowsPerBlock - 1) / kRowsPerBlock, (unsigned)min(a.G, max(a.U, 1)));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
