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
// of split i (per chunk of 64 splits); eight splits' rows are loaded before they are accumulated.
// Groups with more than one split number at most U - 1 (each straddles a unit boundary), so the
// grid's group dimension is capped at U and a workgroup strides over groups; those with one split
// (already final) cost it only their two split pointers.
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kDepth = 8;  // partial rows in flight per lane
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

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  if (!plan_matches(a.plan, a.G, a.U, a.R)) {
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
  // the split pointers of the workgroup's first four groups are requested together
  const int gstep = gridDim.y;
  int p0[4], p1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = min((int)blockIdx.y + i * gstep, a.G - 1);
    p0[i] = a.plan[a.grp_ptr_off + g];
    p1[i] = a.plan[a.grp_ptr_off + g + 1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = (int)blockIdx.y + i * gstep;
    if (g < a.G) {
      const int s0 = __builtin_amdgcn_readfirstlane(p0[i]), s1 = __builtin_amdgcn_readfirstlane(p1[i]);
      if (s1 - s0 != 1) combine_group(a, g, s0, s1);
    }
  }
#pragma unroll 1
  for (int g = (int)blockIdx.y + 4 * gstep; g < a.G; g += gstep) {
    const int s0 = __builtin_amdgcn_readfirstlane(a.plan[a.grp_ptr_off + g]);
    const int s1 = __builtin_amdgcn_readfirstlane(a.plan[a.grp_ptr_off + g + 1]);
    if (s1 - s0 != 1) combine_group(a, g, s0, s1);
  }
}

// The merge of group g's splits [s0, s1) for the workgroup's four rows.
__device__ __forceinline__ void combine_group(const CombineArgs& a, int g, int s0, int s1) {
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
  // LSEs and the first kDepth splits' rows are requested together, so a group with at most kDepth
  // splits costs one memory round trip before its sums; larger groups then load kDepth rows at a
  // time. Rows are accumulated in split order.
  const int64_t row0 = (int64_t)r * kDv + c;
  const uint16_t* po = a.part_o + (int64_t)s0 * a.R * kDv + row0;
  const int64_t po_step = (int64_t)a.R * kDv;
  // (indices past the group's last split repeat it: uniform, branch-free loads whose rows are
  // not accumulated)
  uint4 v[kDepth];
  if (ns > 0) {
#pragma unroll
    for (int q = 0; q < kDepth; ++q) v[q] = *reinterpret_cast<const uint4*>(po + min(q, ns - 1) * po_step);
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
      for (int k = 0; k < nc; k += kDepth) {
        if (sc != s0 || k != 0) {  // the first kDepth rows are already loaded
#pragma unroll
          for (int q = 0; q < kDepth; ++q)
            v[q] = *reinterpret_cast<const uint4*>(po + (sc - s0 + min(k + q, nc - 1)) * po_step);
        }
#pragma unroll
        for (int q = 0; q < kDepth; ++q) {
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
